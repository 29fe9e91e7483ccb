// Host bit-plane packer: uint8 parent codes -> 8 bit-planes in the library's
// chunk-major layout (the Any-Precision overlaid bit-plane form of the
// PagedWeight pages, Core components 1).
//
// Plane p holds bit (7 - p) of every code, so reading planes 0..q-1 yields
// code >> (8 - q).  Word w of a row covers columns 32w..32w+31; column
// 32w + 8P + 2i + h sits at bit 8i + 4h + P.  That in-word order lets the
// device gather assemble four child codes per 32-bit register with one
// and-or per plane (see pw_kernels.hip).  Plane storage is
// [ceil(K/128)][R][4] words.
#include <algorithm>
#include <cstring>
#include <thread>
#include <vector>

#include "pw_internal.h"

namespace pw {

int64_t plane_words(int64_t R, int64_t K) { return ((K + kChunkCols - 1) / kChunkCols) * R * 4; }

static void pack_rows(const uint8_t* codes, int64_t r0, int64_t r1, int64_t R, int64_t K, uint32_t* planes)
{
    const int64_t pw = plane_words(R, K);
    for (int64_t r = r0; r < r1; ++r) {
        const uint8_t* row = codes + r * K;
        for (int64_t w = 0; w < K / 32; ++w) {
            uint32_t word[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            for (int j = 0; j < 32; ++j) {
                const int P = j >> 3, i = (j >> 1) & 3, h = j & 1;
                const int bit = 8 * i + 4 * h + P;
                const uint32_t c = row[32 * w + j];
                for (int p = 0; p < 8; ++p) word[p] |= ((c >> (7 - p)) & 1u) << bit;
            }
            const int64_t at = ((w >> 2) * R + r) * 4 + (w & 3);
            for (int p = 0; p < 8; ++p) planes[p * pw + at] = word[p];
        }
    }
}

void pack_bitplanes(const uint8_t* codes, int64_t R, int64_t K, uint32_t* planes)
{
    const int64_t pw = plane_words(R, K);
    std::memset(planes, 0, sizeof(uint32_t) * 8 * pw);  // zero words of a partial last chunk
    const int64_t work = R * K;
    int nt = (int)std::min<int64_t>(std::max(1u, std::thread::hardware_concurrency()), 16);
    if (work < (int64_t)1 << 20) nt = 1;
    nt = (int)std::min<int64_t>(nt, R);
    if (nt <= 1) {
        pack_rows(codes, 0, R, R, K, planes);
        return;
    }
    std::vector<std::thread> th;
    for (int t = 0; t < nt; ++t) {
        const int64_t r0 = R * t / nt, r1 = R * (t + 1) / nt;
        th.emplace_back(pack_rows, codes, r0, r1, R, K, planes);
    }
    for (auto& x : th) x.join();
}

// Device LUT layout ("slot layout"): LUT_q of a block as [2^q][S] uint32,
// where slot j holds the entries of two rows, row_a(j) in the low and
// row_b(j) in the high 16 bits.  gate_up pairs h-row i's gate row i with its
// up row I + i; down pairs row 64 m + r with row 64 m + 32 + r (r < 32).  S is
// rounded up to a multiple of 64; slots past the block hold zeros.  A decode
// tile of 16 * RG slots is then one contiguous run of 64 * RG bytes per entry.
int lut_slots(int R, int module)
{
    const int s = module == 0 ? R / 2 : (R + 63) / 64 * 32;
    return (s + 63) / 64 * 64;
}

void lut_slot_rows(int R, int module, int j, int* a, int* b)
{
    if (module == 0) {
        *a = j < R / 2 ? j : -1;
        *b = j < R / 2 ? R / 2 + j : -1;
    } else {
        const int ra = 64 * (j / 32) + j % 32;
        *a = ra < R ? ra : -1;
        *b = ra + 32 < R ? ra + 32 : -1;
    }
}

void convert_lut(const uint16_t* luts, int R, int module, int q, uint32_t* out)
{
    const int S = lut_slots(R, module), nc = 1 << q;
    const uint16_t* lq = luts + (size_t)R * (nc - 8);  // LUT_q [R][2^q] in the concatenated k = 3..8 arrays
    for (int j = 0; j < S; ++j) {
        int a, b;
        lut_slot_rows(R, module, j, &a, &b);
        for (int e = 0; e < nc; ++e) {
            const uint32_t lo = a >= 0 ? lq[(size_t)a * nc + e] : 0u;
            const uint32_t hi = b >= 0 ? lq[(size_t)b * nc + e] : 0u;
            out[(size_t)e * S + j] = lo | (hi << 16);
        }
    }
}

}  // namespace pw
