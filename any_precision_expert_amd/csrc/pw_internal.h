// Internal declarations shared by the host ABI layer and the HIP kernels of
// the PagedWeight fused mixed-precision MoE library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pw {

constexpr int kQMin = 3;
constexpr int kQMax = 8;
constexpr int kChunkCols = 128;  // columns per plane chunk (4 words of 32)
constexpr int kLutHalvesPerRow = 8 + 16 + 32 + 64 + 128 + 256;  // LUT_3..LUT_8

// One entry of the device weight page table: a linear block at its committed
// width q.  planes[p] is valid for p < q; lut points at LUT_q in the slot
// layout [2^q][slots] (two rows' fp16 entries per 32-bit slot, see
// convert_lut).
struct alignas(128) BlockDesc {
    const uint32_t* planes[8];
    const uint32_t* lut;
    int32_t q;
    int32_t R;
    int32_t K;
    int32_t nchunks;  // ceil(K / 128)
    int32_t kwords;   // K / 32
    int32_t slots;    // LUT slots (a multiple of 64)
    int32_t pad[8];
};
static_assert(sizeof(BlockDesc) == 128, "page-table entry must be 128 bytes");

// Arguments of the FFN kernels (passed by value).
struct FfnArgs {
    const BlockDesc* table;   // this layer's entries, [(E + 1) * 2]
    const uint16_t* x;        // fp16 [T][H]
    const int32_t* offsets;   // [E + 1]
    const int32_t* sorted;    // [T * k]
    const float* topk_w;      // [T * k]
    uint16_t* h;              // fp16 [T * k + T][hstride]: silu(g) * u rounded to fp16
    float* dout;              // fp32 [T * k + T][H]
    uint16_t* y;              // fp16 [T][H]
    int32_t T, H, I, Is, E, k;
    int32_t n_slots;          // routed slots: min(E, T * k)
    int32_t tiles_routed;     // row tiles per routed block
    int32_t tiles_shared;     // row tiles of the shared block (0 = none)
    int32_t splits_routed;    // K splits per routed row tile (down: >= 1; gate_up: 1)
    int32_t splits_shared;    // K splits per shared row tile
    int32_t hstride;          // max(I, Is)
    int32_t drows;            // rows of one dout split plane: T * k (+ T with a shared expert)
    int32_t rg;               // 32-row groups per workgroup tile: 2 or 4
    int32_t big_wgs;          // rg 4: workgroups taking whole tiles before tiles split in halves (0: all whole)
    int32_t keep_planes;      // decode: ordinary (not nontemporal) plane loads, set when tiles take several passes
    int32_t tok_pass;         // decode: tokens per pass, 8, 16 or 32 (16, 32: 64-row tiles only, routing outside)
    // prefill launches: token tiles of the shared block, and an upper bound
    // on the routed token tiles (sum over experts of ceil(tokens / 512))
    int32_t tok_tiles_shared;
    int32_t tok_tiles_routed;
    // prefill tails: an expert's last (n mod 512) tokens, when fewer than
    // pf_tail, are left out of the GEMM tiles and taken by the decode launches,
    // which then run on those tails only (0: no tails)
    int32_t pf_tail;
    // routing inside the decode gate_up launch (logits non-null; T * k <=
    // kLayerRouteMaxAssign): every routed workgroup routes and sorts the batch
    // in LDS, and one of them writes the results that the down and combine
    // launches read (offsets, sorted, topk_w above point at the same buffers)
    const float* logits;
    int32_t* idx_out;
    float* w_out;
    int32_t* offsets_out;
    int32_t* sorted_out;
    // routing-mass accumulator row of this layer ([E] fp64) or null
    double* mass;
};

// Most assignments (T * k) a gate_up launch routes by itself.
constexpr int kLayerRouteMaxAssign = 64;


// Tokens per decode pass: the smallest of 8, 16 and 32 that covers the
// largest token count a work unit is expected to hold -- the shared expert's
// T, or for routed experts the mean T k / E plus two standard deviations of a
// Poisson count.  Wider passes decode each weight once for more tokens (the
// MFMA's B operand has 32 token columns either way) but cost more per pass:
// on a Mixtral-shaped layer with all units in one pass, 16-token passes were
// 5% and 32-token passes 14% slower than 8-token ones; batch 32 (12 tokens on
// the fullest expert) 0.40 -> 0.30 ms with 16-token passes, batch 64 0.41 ->
// 0.33 ms and batch 128 0.66 -> 0.45 ms with 32-token passes; a
// Qwen-shaped layer (shared expert) 0.068 -> 0.062 ms at batch 12 with 16,
// 0.21 -> 0.12 ms at batch 64 with 32.
inline double decode_unit_tokens(int T, int k, int E, int I_shared)
{
    const double a = (double)T * k / E;
    const double m = a + 2.0 * __builtin_sqrt(a);
    return I_shared > 0 && T > m ? (double)T : m;
}

inline int decode_tok_pass(int T, int k, int E, int I_shared)
{
    const double m = decode_unit_tokens(T, k, E, I_shared);
    return m <= 8.0 ? 8 : m <= 16.0 ? 16 : 32;
}

// Decode launches load planes with ordinary loads (which the MALL keeps)
// instead of nontemporal ones when the fullest units are expected to take a
// second pass and re-read their planes (Mixtral-shaped batch 128 0.469 ->
// 0.443 ms).  With one pass, nontemporal loads are faster (ordinary loads
// made the Qwen-shaped step 4% and Mixtral-shaped batches of 1-48 1-3%
// slower).
inline bool keep_planes(int T, int k, int E, int I_shared, int tok_pass)
{
    return decode_unit_tokens(T, k, E, I_shared) > (double)tok_pass;
}

// Tokens per call from which the prefill GEMM path runs.
constexpr int kPrefillMinT = 256;
// Tokens per prefill GEMM tile, and the bound below which an expert's tail
// (its n mod 512 tokens past the last whole tile) goes to the decode launches
// instead of a GEMM tile: a GEMM tile decodes the expert's weights once
// whatever its token count, a decode pass streams them once per 32 tokens.
// Mixtral-shaped prefill, same box: a tail tile cost ~97 us of gate_up GEMM and
// ~40 us of down GEMM, a 32-token decode pass ~27 + ~14 us, so up to three
// passes (96 tokens) the decode launches are cheaper; with the three 24-32
// token tails of uniform routing the layer step went 4.06-4.08 -> 3.84-3.88 ms.
constexpr int kPrefillTokTile = 512;
constexpr int kPrefillTail = 96;

// 32-row groups per workgroup tile (two share one LUT set; four use both
// halves of the LUT slots): gate_up tiles hold 16 * rg gate rows and their up
// rows, down tiles 32 * rg output rows.
constexpr int kGateUpRowGroups = 4;
constexpr int kDownRowGroups = 2;

// K splits of a down-projection row tile, so long K ranges spread over the
// chip: at most 16 128-column chunks per workgroup (four per wave) up to 64
// chunks, at most 32 beyond.  Each split stages the tile's whole LUT again,
// so for long K (Mixtral-shaped, 112 chunks) fewer, longer splits win (down
// -10..-18% at batch 1-16), while a short K (the Qwen-shaped shared expert,
// 44 chunks) needs the parallelism of 16-chunk splits.
inline int down_splits(int K)
{
    const int nchunks = (K + kChunkCols - 1) / kChunkCols;
    const int per = nchunks > 64 ? 32 : 16;
    return nchunks <= per ? 1 : (nchunks + per - 1) / per;
}

// K splits of the routed down tiles of a decode launch: the fewest (powers of
// two, at most down_splits(K)) that keep ~1.75 workgroups per CU busy, counting
// the row tiles of the experts a batch is expected to activate (an expert is
// idle with probability (1 - k/E)^T).  Each split re-stages the tile's LUT and
// pays the tile's start-up chain, so splits only pay where there are too few
// active tiles to fill the chip.  Mixtral-shaped down (112 chunks, 64 row
// tiles), 4 / 2 / 1 splits: batch 1 23.5 / 25.1 / 41.2 us, batch 4 53.8 /
// 46.8 / 58.1, batch 16 76.2 / 64.4 / 64.2, batch 64 93.1 / 81.7 / 75.8.
inline int down_splits_routed(int K, int T, int k, int E, int tiles, int cus)
{
    const int cap = down_splits(K);
    const double idle = __builtin_pow(1.0 - (double)k / E, (double)T);
    const double active_tiles = (double)tiles * E * (1.0 - idle);
    int s = 1;
    while (s < cap && active_tiles * s < 1.75 * cus) s *= 2;
    return s < cap ? s : cap;
}

// Workspace carve-up for T tokens (byte offsets, 256-aligned): h as fp16
// [T*k (+T)][max(I, Is)], then the per-split down outputs
// [splits][T*k (+T)][H] fp32.
struct WsLayout {
    size_t h, dout, total;
};
WsLayout ws_layout(int T, int k, int H, int I, int Is);

// Launchers (return the launch's hipError_t).
// Timing of one launch by its own dispatch (hipExtLaunchKernelGGL start /
// stop events): while launch_events points at an unused pair, the next kernel
// launched on this thread records it and sets `used`.  The events then bracket
// the kernel alone, not the queue packets around it.
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
    bool used = false;
};
extern thread_local LaunchEvents* launch_events;

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                             hipStream_t s);
hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                          int32_t* sorted, hipStream_t s);
// one workgroup routes and sorts (T * k <= kFusedMaxAssign)
constexpr int kFusedMaxAssign = 4096;
hipError_t launch_route_permute(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                                int32_t* offsets, int32_t* sorted, hipStream_t s);
hipError_t launch_gate_up(const FfnArgs& a, hipStream_t s);  // routes first when a.logits is set
hipError_t launch_down(const FfnArgs& a, hipStream_t s);
hipError_t launch_prefill(const FfnArgs& a, int module, hipStream_t s);
hipError_t launch_combine(const FfnArgs& a, hipStream_t s);
// mass[e] += sum of w[sorted[p]] over p in [offsets[e], offsets[e+1]), fp64 in
// that order (one workgroup)
hipError_t launch_routing_mass(const int32_t* offsets, const int32_t* sorted, const float* w, int E, double* mass,
                               hipStream_t s);
hipError_t launch_fill_f64(double* p, int64_t n, hipStream_t s);
// Decode of one block as an FFN path runs it (path: 0 decode contraction
// with 128-row gate_up / down tiles (RG = 4), 1 with 64-row tiles (RG = 2),
// 2 prefill decoder, 3 64-row tiles of 16-token passes); codes_out uint8
// [R][K] and / or w_out fp16 [R][K].
hipError_t launch_debug_decode(const BlockDesc* entry, int module, int R, int path, uint8_t* codes_out,
                               uint16_t* w_out, hipStream_t s);

// One copy of a width change (device-side addresses, bytes a multiple of 16).
struct CopyDesc {
    const void* src;
    void* dst;
    uint64_t bytes;
};
// The copies of list[0..n) (the list itself in pinned host memory), one
// launch: from pinned host memory by a few workgroups (pull), or device to
// device as a short burst over many workgroups (scatter).
hipError_t launch_pull_copy(const CopyDesc* list, int n, hipStream_t s);
hipError_t launch_scatter_copy(const CopyDesc* list, int n, hipStream_t s);
// table[ids[i]] = descs[i] for i < n (ids and descs in pinned host memory).
hipError_t launch_scatter_desc(BlockDesc* table, const int32_t* ids, const BlockDesc* descs, int n, hipStream_t s);

// Library-held workspace of pw_moe_layer_noalloc (pw_kernels.hip): its size,
// and its device address on `device`, looked up once per device (call with
// that device current).
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;
hipError_t static_scratch(int device, void** out);

// Host packer (pw_pack.cpp).
void pack_bitplanes(const uint8_t* codes, int64_t R, int64_t K, uint32_t* planes);
int64_t plane_words(int64_t R, int64_t K);
// Device LUT slot layout (pw_pack.cpp): slots of a block, the two rows of a
// slot (-1 past the block), and LUT_q of the concatenated k = 3..8 host
// arrays [R][2^k] rewritten as [2^q][slots] uint32.
int lut_slots(int R, int module);
void lut_slot_rows(int R, int module, int j, int* a, int* b);
void convert_lut(const uint16_t* luts, int R, int module, int q, uint32_t* out);

}  // namespace pw
