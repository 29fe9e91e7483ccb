// HIP kernels (gfx950 / CDNA4) of the PagedWeight fused mixed-precision MoE
// path: top-k routing, the stable permutation by expert, the bit-plane
// streaming gate_up / down contractions with per-row LUTs, and the
// gate-weighted combine.
//
// Method (PagedWeight pages, "Technical summary: PagedWeight", Core
// components 1 and 3): each per-expert linear block is stored as overlaid
// bit-planes with per-row LUTs and read at its own committed width q inside
// one fused MoE operation.  The parent code has 8 bits; the width-q child
// code is code >> (8 - q) = the top q planes; the weight is LUT_q[row][code].
//
// Decode-sized contraction ("bit-plane-streaming GEMV"): one workgroup owns 64
// weight rows (one per lane) and splits K across its 8 waves.  Each lane
// streams its row's q plane words with 16-byte loads ([chunk][row][4] layout:
// 64 lanes read 1 KB contiguous), assembles child codes with a register-level
// bit gather, looks weights up in the LDS copy of its row's LUT and
// accumulates against fp16 activations held in scalar registers with
// v_dot2_f32_f16 (fp32 accumulation).  The LUT lives in LDS as [code][lane]
// 32-bit slots so a wave's 64 look-ups hit 32 distinct banks per half-wave;
// for q <= 4 a pair table [code_a | code_b << q][lane] returns two weights
// (a packed half2) per look-up.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "pw_internal.h"

namespace pw {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(4))) const uint32_t* cu32p;  // scalar-loadable
typedef __attribute__((address_space(1))) const u32x4* gu32x4p;    // global (not flat)

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kLutBytes = 65536;  // largest LDS LUT: 256 slots x 64 lanes x 4 B
constexpr int kGemvLdsWords = kLutBytes / 4 + kWaves * 4 * 64;  // LUT + cross-wave reduction
constexpr int kDebugLdsWords = kLutBytes / 4 + 16 * 64;        // LUT + pair staging

// ---------------------------------------------------------------- bit gather

__device__ __forceinline__ uint32_t rotl(uint32_t x, int n)
{
    return __builtin_amdgcn_alignbit(x, x, (32 - (n & 31)) & 31);
}
__device__ __forceinline__ uint32_t rotr(uint32_t x, int n) { return __builtin_amdgcn_alignbit(x, x, n & 31); }

// 0x01010101 rotated left by n: one bit in each byte, at position n mod 8.
__host__ __device__ constexpr uint32_t rep_bit(int n) { return 0x01010101u << (((n % 8) + 8) % 8); }

// Gathered child codes of one 32-column plane word set (W[p] = word of plane p).
//  single (q >= 5): r[2P + h] byte i = code of column 8P + 2i + h
//  pair   (q <= 4): r[P]      byte i = code(8P + 2i) | code(8P + 2i + 1) << q
template <int Q>
struct Gathered {
    static constexpr int N = Q <= 4 ? 4 : 8;
    uint32_t r[N];
};

// In the stored word, column 8P + 2i + h is at bit 8i + 4h + P.  Rotating plane
// p left by (q - 1 - p) moves every bit of that plane by the same amount, so a
// single and-or per (plane, register) drops its bit of four columns into the
// right position of four bytes at once; one final rotate per register aligns
// the bytes.
template <int Q>
__device__ __forceinline__ void gather(const uint32_t (&W)[Q], Gathered<Q>& g)
{
    uint32_t A[Q];
#pragma unroll
    for (int p = 0; p < Q; ++p) A[p] = rotl(W[p], Q - 1 - p);
    if constexpr (Q <= 4) {
        uint32_t B[Q];
#pragma unroll
        for (int p = 0; p < Q; ++p) B[p] = rotl(W[p], 2 * Q - 5 - p);
#pragma unroll
        for (int P = 0; P < 4; ++P) {
            uint32_t acc = 0;
#pragma unroll
            for (int p = 0; p < Q; ++p) {
                acc |= A[p] & rep_bit(P + Q - 1 - p);
                acc |= B[p] & rep_bit(P + 2 * Q - 1 - p);
            }
            g.r[P] = rotr(acc, P);
        }
    } else {
#pragma unroll
        for (int P = 0; P < 4; ++P) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t acc = 0;
#pragma unroll
                for (int p = 0; p < Q; ++p) acc |= A[p] & rep_bit(4 * h + P + Q - 1 - p);
                g.r[2 * P + h] = rotr(acc, 4 * h + P);
            }
        }
    }
}

// LDS byte address of byte i of `codes`: (code << 8) | lane_off.
__device__ __forceinline__ uint32_t lut_addr(uint32_t codes, uint32_t lane_off, int i)
{
    return __builtin_amdgcn_perm(codes, lane_off, 0x0c0c0000u | ((4u + (uint32_t)i) << 8));
}

// Weights of the 32 columns as 16 half2 pairs: w2[4P + i] = (W[8P+2i], W[8P+2i+1]).
template <int Q>
__device__ __forceinline__ void lookup(const Gathered<Q>& g, uint32_t lane_off, const char* lutb,
                                       h2 (&w2)[16])
{
#pragma unroll
    for (int P = 0; P < 4; ++P) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (Q <= 4) {
                w2[4 * P + i] = *(const h2*)(lutb + lut_addr(g.r[P], lane_off, i));
            } else {
                h2 v;
                v.x = *(const _Float16*)(lutb + lut_addr(g.r[2 * P], lane_off, i));
                v.y = *(const _Float16*)(lutb + lut_addr(g.r[2 * P + 1], lane_off, i));
                w2[4 * P + i] = v;
            }
        }
    }
}

// LUT_q of this lane's row -> LDS slots [entry][lane] (32-bit each).
// Single (q >= 5): entry = code, low half = LUT[code].  Pair (q <= 4):
// entry = a | b << q, value = LUT[a] | LUT[b] << 16; the single table is
// staged first in `stage` (2^q x 64 slots) and the caller's barrier follows.
template <int Q>
__device__ __forceinline__ void load_lut(uint32_t* lds, uint32_t* stage, const uint16_t* lut, int row,
                                         bool valid, int lane, int wave, int nwaves)
{
    constexpr int NC = 1 << Q;
    uint32_t* single = Q <= 4 ? stage : lds;
    gu32x4p src = (gu32x4p)(uintptr_t)(lut + (size_t)row * NC);
    for (int c8 = wave; c8 < NC / 8; c8 += nwaves) {
        u32x4 u = valid ? src[c8] : u32x4{0, 0, 0, 0};
        const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) single[((8 * c8 + j) << 6) | lane] = (w4[j >> 1] >> (16 * (j & 1))) & 0xffffu;
    }
    if constexpr (Q <= 4) {
        __syncthreads();
        for (int e = wave; e < NC * NC; e += nwaves) {
            const int ea = e & (NC - 1), eb = e >> Q;
            lds[(e << 6) | lane] = single[(ea << 6) | lane] | (single[(eb << 6) | lane] << 16);
        }
    }
}

__device__ __forceinline__ uint4 load_planes_chunk(const uint32_t* plane, int c, int R, int row, bool valid)
{
    if (!valid) return make_uint4(0, 0, 0, 0);
    const u32x4 v = __builtin_nontemporal_load((gu32x4p)(uintptr_t)plane + ((size_t)c * R + row));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int ww)
{
    return ww == 0 ? v.x : ww == 1 ? v.y : ww == 2 ? v.z : v.w;
}

__device__ __forceinline__ float dot2(h2 a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(a, __builtin_bit_cast(h2, b), c, false);
}

// ---------------------------------------------------------------- routing

__global__ void __launch_bounds__(256) route_topk_kernel(const float* __restrict__ logits, int T, int E,
                                                         int k, int32_t* __restrict__ idx,
                                                         float* __restrict__ w)
{
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T) return;
    float v[8];
    int id[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        v[j] = 0.0f;
        id[j] = -1;
    }
    const float* l = logits + (size_t)t * E;
    for (int e = 0; e < E; ++e) {
        // insert (l[e], e) by the key (value descending, index ascending); the
        // displaced entry moves down one slot at a time, branch-free
        float cv = l[e];
        int ci = e;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool take = j < k && ci >= 0 && (id[j] < 0 || cv > v[j] || (cv == v[j] && ci < id[j]));
            const float nv = take ? cv : v[j];
            const int ni = take ? ci : id[j];
            cv = take ? v[j] : cv;
            ci = take ? id[j] : ci;
            v[j] = nv;
            id[j] = ni;
        }
    }
    const float m = v[0];
    float ex[8], s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        ex[j] = j < k ? expf(v[j] - m) : 0.0f;
        s += ex[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (j < k) {
            idx[(size_t)t * k + j] = id[j];
            w[(size_t)t * k + j] = ex[j] / s;
        }
    }
}

// One workgroup: count per expert, exclusive scan, then a stable placement of
// assignments chunk by chunk (rank inside a wave from a ballot match, rank
// across waves from per-wave counts).
__global__ void __launch_bounds__(1024) permute_kernel(const int32_t* __restrict__ idx, int n, int E,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ sorted)
{
    __shared__ int cnt[256];
    __shared__ int base[256];
    __shared__ int wcnt[16][256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int e = tid; e < E; e += 1024) cnt[e] = 0;
    __syncthreads();
    for (int a = tid; a < n; a += 1024) {
        const int e = idx[a];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    if (tid == 0) {
        int s = 0;
        for (int e = 0; e < E; ++e) {
            base[e] = s;
            offsets[e] = s;
            s += cnt[e];
        }
        offsets[E] = s;
    }
    __syncthreads();
    for (int a0 = 0; a0 < n; a0 += 1024) {
        for (int i = tid; i < 16 * 256; i += 1024) (&wcnt[0][0])[i] = 0;
        __syncthreads();
        const int a = a0 + tid;
        int e = a < n ? idx[a] : 511;
        if (e < 0 || e >= E) e = 511;
        unsigned long long m = ~0ull;
#pragma unroll
        for (int b = 0; b < 9; ++b) {
            const int bit = (e >> b) & 1;
            const unsigned long long bal = __ballot(bit);
            m &= bit ? bal : ~bal;
        }
        const int rank = __popcll(m & ((1ull << lane) - 1ull));
        const int leader = __ffsll((long long)m) - 1;
        if (lane == leader && e < E) wcnt[wave][e] = __popcll(m);
        __syncthreads();
        if (e < E) {
            int pre = 0;
            for (int w = 0; w < wave; ++w) pre += wcnt[w][e];
            sorted[base[e] + pre + rank] = a;
        }
        __syncthreads();
        for (int e2 = tid; e2 < E; e2 += 1024) {
            int s = 0;
            for (int w = 0; w < 16; ++w) s += wcnt[w][e2];
            base[e2] += s;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- FFN GEMV

// MODE 0: gate_up. 64 lanes = 32 gate rows + the 32 matching up rows; input
//         x (fp16); epilogue h = silu(g) * u stored as fp16 hi + fp16 lo.
// MODE 1: down. 64 lanes = 64 output rows; input h = hi + lo; epilogue writes
//         the fp32 expert output of each assignment.
template <int MODE>
struct ModeTraits {
    static constexpr int TT = MODE == 0 ? 4 : 2;  // tokens per pass
};

template <int MODE, int Q>
__device__ void gemv_block(const FfnArgs& a, const BlockDesc* __restrict__ bd, bool shared, int p0,
                           int ntok, int tile, uint32_t* lds)
{
    constexpr int TT = ModeTraits<MODE>::TT;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps K offsets scalar
    const int R = bd->R;
    const int nchunks = bd->nchunks, kwords = bd->kwords;
    int row;
    bool valid;
    if (MODE == 0) {
        const int Iblk = R >> 1;
        const int i = tile * 32 + (lane & 31);
        valid = i < Iblk;
        row = lane < 32 ? i : Iblk + i;
    } else {
        row = tile * 64 + lane;
        valid = row < R;
    }
    load_lut<Q>(lds, lds + kLutBytes / 4, bd->lut, row, valid, lane, wave, kWaves);
    __syncthreads();

    const char* lutb = (const char*)lds;
    float* red = (float*)(lds + kLutBytes / 4);
    const uint32_t lane_off = (uint32_t)lane * 4u;
    const uint32_t* planes[Q];
#pragma unroll
    for (int p = 0; p < Q; ++p) planes[p] = bd->planes[p];
    const int TK = a.T * a.k;

    for (int t0 = 0; t0 < ntok; t0 += TT) {
        const int nt = min(TT, ntok - t0);
        cu32p in_hi[TT];
        cu32p in_lo[TT];
#pragma unroll
        for (int j = 0; j < TT; ++j) {
            const int jj = t0 + min(j, nt - 1);
            if (MODE == 0) {
                const int tok = __builtin_amdgcn_readfirstlane(shared ? jj : a.sorted[p0 + jj] / a.k);
                in_hi[j] = (cu32p)(uintptr_t)(a.x + (size_t)tok * a.H);
                in_lo[j] = in_hi[j];
            } else {
                const int hrow = __builtin_amdgcn_readfirstlane(shared ? TK + jj : p0 + jj);
                in_hi[j] = (cu32p)(uintptr_t)(a.h_hi + (size_t)hrow * a.hstride);
                in_lo[j] = (cu32p)(uintptr_t)(a.h_lo + (size_t)hrow * a.hstride);
            }
        }
        float acc[TT];
#pragma unroll
        for (int j = 0; j < TT; ++j) acc[j] = 0.0f;

        for (int c = wave; c < nchunks; c += kWaves) {
            uint4 pv[Q];
#pragma unroll
            for (int p = 0; p < Q; ++p) pv[p] = load_planes_chunk(planes[p], c, R, row, valid);
            const int nw = min(4, kwords - 4 * c);
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) {
                if (ww < nw) {
                    uint32_t W[Q];
#pragma unroll
                    for (int p = 0; p < Q; ++p) W[p] = word_of(pv[p], ww);
                    Gathered<Q> g;
                    gather<Q>(W, g);
                    h2 w2[16];
                    lookup<Q>(g, lane_off, lutb, w2);
                    const int col2 = c * 64 + ww * 16;
#pragma unroll
                    for (int j = 0; j < TT; ++j) {
                        if (j < nt) {
#pragma unroll
                            for (int i = 0; i < 16; ++i) acc[j] = dot2(w2[i], in_hi[j][col2 + i], acc[j]);
                            if (MODE == 1) {
#pragma unroll
                                for (int i = 0; i < 16; ++i) acc[j] = dot2(w2[i], in_lo[j][col2 + i], acc[j]);
                            }
                        }
                    }
                }
            }
        }

#pragma unroll
        for (int j = 0; j < TT; ++j) red[(wave * TT + j) * 64 + lane] = acc[j];
        __syncthreads();
        if (wave == 0) {
            for (int j = 0; j < nt; ++j) {
                if (MODE == 0) {
                    if (lane < 32) {
                        float g = 0.0f, u = 0.0f;
#pragma unroll
                        for (int w = 0; w < kWaves; ++w) {
                            g += red[(w * TT + j) * 64 + lane];
                            u += red[(w * TT + j) * 64 + lane + 32];
                        }
                        const float h = g / (1.0f + __expf(-g)) * u;
                        const _Float16 hi = (_Float16)h;
                        const _Float16 lo = (_Float16)(h - (float)hi);
                        if (valid) {
                            const int hrow = shared ? TK + t0 + j : p0 + t0 + j;
                            const size_t o = (size_t)hrow * a.hstride + tile * 32 + lane;
                            a.h_hi[o] = __builtin_bit_cast(uint16_t, hi);
                            a.h_lo[o] = __builtin_bit_cast(uint16_t, lo);
                        }
                    }
                } else {
                    float d = 0.0f;
#pragma unroll
                    for (int w = 0; w < kWaves; ++w) d += red[(w * TT + j) * 64 + lane];
                    if (valid) {
                        const int orow = shared ? TK + t0 + j : a.sorted[p0 + t0 + j];
                        a.dout[(size_t)orow * a.H + row] = d;
                    }
                }
            }
        }
        __syncthreads();
    }
}

template <int MODE>
__global__ void __launch_bounds__(kThreads) ffn_gemv_kernel(FfnArgs a)
{
    __shared__ uint32_t lds[kGemvLdsWords];
    const int wg = blockIdx.x;
    const int routed_wgs = a.n_slots * a.tiles_routed;
    bool shared;
    int tile, p0, ntok, slot_expert;
    if (wg < routed_wgs) {
        shared = false;
        const int slot = wg / a.tiles_routed;
        tile = wg - slot * a.tiles_routed;
        // the slot-th expert with at least one routed assignment
        int e = -1, cnt = 0;
        for (int ee = 0; ee < a.E; ++ee) {
            if (a.offsets[ee + 1] > a.offsets[ee]) {
                if (cnt == slot) {
                    e = ee;
                    break;
                }
                ++cnt;
            }
        }
        if (e < 0) return;
        p0 = a.offsets[e];
        ntok = a.offsets[e + 1] - p0;
        slot_expert = e;
    } else {
        shared = true;
        tile = wg - routed_wgs;
        p0 = 0;
        ntok = a.T;
        slot_expert = a.E;
    }
    const BlockDesc* bd = a.table + (slot_expert * 2 + MODE);
    switch (bd->q) {
        case 3: gemv_block<MODE, 3>(a, bd, shared, p0, ntok, tile, lds); break;
        case 4: gemv_block<MODE, 4>(a, bd, shared, p0, ntok, tile, lds); break;
        case 5: gemv_block<MODE, 5>(a, bd, shared, p0, ntok, tile, lds); break;
        case 6: gemv_block<MODE, 6>(a, bd, shared, p0, ntok, tile, lds); break;
        case 7: gemv_block<MODE, 7>(a, bd, shared, p0, ntok, tile, lds); break;
        case 8: gemv_block<MODE, 8>(a, bd, shared, p0, ntok, tile, lds); break;
        default: break;
    }
}

__global__ void __launch_bounds__(256) combine_kernel(FfnArgs a)
{
    const size_t n = (size_t)a.T * a.H;
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int t = (int)(i / a.H), o = (int)(i - (size_t)t * a.H);
    float s = 0.0f;
    for (int j = 0; j < a.k; ++j) s += a.topk_w[t * a.k + j] * a.dout[((size_t)t * a.k + j) * a.H + o];
    if (a.tiles_shared) s += a.dout[((size_t)a.T * a.k + t) * a.H + o];
    a.y[i] = __builtin_bit_cast(uint16_t, (_Float16)s);
}

// ---------------------------------------------------------------- debug export

// Same LUT staging, gather and look-up as the FFN: one wave per 64 rows.
template <int Q>
__device__ void debug_block(const BlockDesc* __restrict__ bd, int R, int K, uint8_t* codes_out,
                            uint16_t* w_out, uint32_t* lds)
{
    const int lane = threadIdx.x;
    const int row = blockIdx.x * 64 + lane;
    const bool valid = row < R;
    load_lut<Q>(lds, lds + kLutBytes / 4, bd->lut, row, valid, lane, 0, 1);
    __syncthreads();
    const char* lutb = (const char*)lds;
    const uint32_t lane_off = (uint32_t)lane * 4u;
    for (int c = 0; c < bd->nchunks; ++c) {
        uint4 pv[Q];
#pragma unroll
        for (int p = 0; p < Q; ++p) pv[p] = load_planes_chunk(bd->planes[p], c, R, row, valid);
        for (int ww = 0; ww < 4 && 4 * c + ww < bd->kwords; ++ww) {
            uint32_t W[Q];
#pragma unroll
            for (int p = 0; p < Q; ++p) W[p] = word_of(pv[p], ww);
            Gathered<Q> g;
            gather<Q>(W, g);
            h2 w2[16];
            lookup<Q>(g, lane_off, lutb, w2);
            if (!valid) continue;
            const size_t base = (size_t)row * K + 32 * (4 * c + ww);
#pragma unroll
            for (int P = 0; P < 4; ++P) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    uint32_t ca, cb;
                    if constexpr (Q <= 4) {
                        const uint32_t pr = (g.r[P] >> (8 * i)) & 0xffu;
                        ca = pr & ((1u << Q) - 1u);
                        cb = pr >> Q;
                    } else {
                        ca = (g.r[2 * P] >> (8 * i)) & 0xffu;
                        cb = (g.r[2 * P + 1] >> (8 * i)) & 0xffu;
                    }
                    const int col = 8 * P + 2 * i;
                    if (codes_out) {
                        codes_out[base + col] = (uint8_t)ca;
                        codes_out[base + col + 1] = (uint8_t)cb;
                    }
                    if (w_out) {
                        const uint32_t pr = __builtin_bit_cast(uint32_t, w2[4 * P + i]);
                        w_out[base + col] = (uint16_t)(pr & 0xffffu);
                        w_out[base + col + 1] = (uint16_t)(pr >> 16);
                    }
                }
            }
        }
    }
}

__global__ void __launch_bounds__(64) debug_decode_kernel(const BlockDesc* __restrict__ bd, int R, int K,
                                                          uint8_t* codes_out, uint16_t* w_out)
{
    __shared__ uint32_t lds[kDebugLdsWords];
    switch (bd->q) {
        case 3: debug_block<3>(bd, R, K, codes_out, w_out, lds); break;
        case 4: debug_block<4>(bd, R, K, codes_out, w_out, lds); break;
        case 5: debug_block<5>(bd, R, K, codes_out, w_out, lds); break;
        case 6: debug_block<6>(bd, R, K, codes_out, w_out, lds); break;
        case 7: debug_block<7>(bd, R, K, codes_out, w_out, lds); break;
        case 8: debug_block<8>(bd, R, K, codes_out, w_out, lds); break;
        default: break;
    }
}

// ---------------------------------------------------------------- launchers


hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w, hipStream_t s)
{
    hipLaunchKernelGGL(route_topk_kernel, dim3((T + 255) / 256), dim3(256), 0, s, logits, T, E, k, idx, w);
    return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets, int32_t* sorted,
                          hipStream_t s)
{
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(1024), 0, s, idx, T * k, E, offsets, sorted);
    return hipGetLastError();
}

hipError_t launch_gate_up(const FfnArgs& a, hipStream_t s)
{
    const int grid = a.n_slots * a.tiles_routed + a.tiles_shared;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(ffn_gemv_kernel<0>, dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_down(const FfnArgs& a, hipStream_t s)
{
    const int grid = a.n_slots * a.tiles_routed + a.tiles_shared;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(ffn_gemv_kernel<1>, dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_combine(const FfnArgs& a, hipStream_t s)
{
    const size_t n = (size_t)a.T * a.H;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_debug_decode(const BlockDesc* entry, int R, int K, uint8_t* codes_out, uint16_t* w_out,
                               hipStream_t s)
{
    hipLaunchKernelGGL(debug_decode_kernel, dim3((R + 63) / 64), dim3(64), 0, s, entry, R, K, codes_out,
                       w_out);
    return hipGetLastError();
}

}  // namespace pw
