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
// Contraction: one 8-wave workgroup owns a 64-row tile of one block (gate_up
// pairs 32 gate rows with the matching 32 up rows).  Waves 0-3 take row group
// 0, waves 4-7 row group 1; the four waves of a group split K by 128-column
// chunks.  Lane (row, half) of a wave streams two words of each of its row's q
// planes per chunk ([chunk][row][4] layout: 512 contiguous bytes per wave and
// plane), assembles child codes with a register-level bit gather, looks the
// weights up in the LDS copy of the rows' LUTs and feeds them as the A operand
// of v_mfma_f32_32x32x16_f16, with up to 32 tokens as B (fp32 accumulation).
// Each weight is decoded once per 32 tokens.  The LUT lives in LDS as
// [code][64 slots] 32-bit slots so a half-wave's 32 look-ups hit 32 distinct
// banks; for q <= 4 a pair table [code_a | code_b << q] returns two weights (a
// packed half2) per look-up.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "pw_internal.h"

namespace pw {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(4))) const uint32_t* cu32p;  // scalar-loadable
typedef __attribute__((address_space(1))) const u32x4* gu32x4p;    // global (not flat)

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kLutBytes = 65536;  // largest LDS LUT: 256 slots x 64 lanes x 4 B
constexpr int kStageWords = 16 * 64;  // pair-table staging (single LUT of q <= 4)
// LUT + eight 2 KB per-wave activation slices (which also hold the pair-table
// staging and the cross-wave reduction): 80 KB, two 8-wave workgroups per CU.
constexpr int kGemvLdsWords = kLutBytes / 4 + kWaves * 512;

// ---------------------------------------------------------------- bit gather

__device__ __forceinline__ uint32_t rotl(uint32_t x, int n)
{
    return __builtin_amdgcn_alignbit(x, x, (32 - (n & 31)) & 31);
}
__device__ __forceinline__ uint32_t rotr(uint32_t x, int n) { return __builtin_amdgcn_alignbit(x, x, n & 31); }

// 0x01010101 rotated left by n: one bit in each byte, at position n mod 8.
__host__ __device__ constexpr int rep_index(int n) { return ((n % 8) + 8) % 8; }

// The eight masks 0x01010101 << s live in scalar registers: a VOP3 and-or on
// gfx9 cannot encode a 32-bit literal, and with the mask in an SGPR every
// (plane, register) step of the gather is a single v_and_or_b32.
struct RepMasks {
    uint32_t m[8];
};

// acc | (a & m) in one v_bitop3_b32 (truth table 0xEC = (S0 & S2) | S1).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t acc)
{
    return (uint32_t)__builtin_amdgcn_bitop3_b32((int)a, (int)acc, (int)m, 0xEC);
}
#define PW_SMASK(s) asm("s_mov_b32 %0, %1" : "=s"(r.m[s]) : "n"(0x01010101u << (s)))
__device__ __forceinline__ RepMasks make_masks()
{
    RepMasks r;
    PW_SMASK(0);
    PW_SMASK(1);
    PW_SMASK(2);
    PW_SMASK(3);
    PW_SMASK(4);
    PW_SMASK(5);
    PW_SMASK(6);
    PW_SMASK(7);
    return r;
}
#undef PW_SMASK

// Child codes of one plane word set by an 8 x 8 bit transpose per byte: with
// row r = plane q - 1 - r (rows q..7 zero), byte i of row r holds bit r of the
// codes of columns 8P + 2i + h at bit 4h + P; three swap stages (4-, 2- and
// 1-bit blocks between rows 4, 2 and 1 apart) leave in row 4h + P, byte i,
// the child code of column 8P + 2i + h.  Each swap is two shifts and two
// bit-selects (v_bitop3); swaps against a row still known to be zero cost
// less.  X[P] / X[4 + P] are the two code registers of MFMA step P.
template <int Q>
__device__ __forceinline__ void transpose_codes(const uint32_t (&W)[Q], uint32_t (&X)[8], uint32_t zero = 0u)
{
    // rows q..7 start as `zero`: a caller that passes a zero the compiler
    // cannot see keeps every swap a plain bit-select pair
#pragma unroll
    for (int r = 0; r < 8; ++r) X[r] = r < Q ? W[Q - 1 - r] : zero;
    auto swap = [](uint32_t& a, uint32_t& b, int sh, uint32_t lo) {
        // a keeps its low bits of each group and takes b's low bits above them;
        // b keeps its high bits and takes a's high bits below them
        const uint32_t na = (a & lo) | ((b << sh) & ~lo);
        const uint32_t nb = (b & ~lo) | ((a >> sh) & lo);
        a = na;
        b = nb;
    };
#pragma unroll
    for (int r = 0; r < 4; ++r) swap(X[r], X[r + 4], 4, 0x0F0F0F0Fu);
    swap(X[0], X[2], 2, 0x33333333u);
    swap(X[1], X[3], 2, 0x33333333u);
    swap(X[4], X[6], 2, 0x33333333u);
    swap(X[5], X[7], 2, 0x33333333u);
#pragma unroll
    for (int r = 0; r < 8; r += 2) swap(X[r], X[r + 1], 1, 0x55555555u);
}

// LDS byte address of byte i of `codes`: (code << 8) | lane_off.
__device__ __forceinline__ uint32_t lut_addr(uint32_t codes, uint32_t lane_off, int i)
{
    return __builtin_amdgcn_perm(codes, lane_off, 0x0c0c0000u | ((4u + (uint32_t)i) << 8));
}

// Code gather of one plane word set W[p] (word of plane p), step by step.
// In the stored word, column 8P + 2i + h is at bit 8i + 4h + P.  Rotating
// plane p left by (q - 1 - p) moves every bit of that plane by the same
// amount, so one and-or per (plane, code register) drops its bit of four
// columns into the right position of four bytes at once, and one final rotate
// per register aligns the bytes.  The planes are rotated once (Rot); each
// MFMA step P then assembles only its own code register(s) and looks up its
// 8 weights, which keeps few registers live.  Pair tables (two weights per
// look-up) gather code(8P + 2i) | code(8P + 2i + 1) << q into byte i.
template <int Q, bool PAIR>
struct Rot {
    uint32_t A[Q];
    uint32_t B[PAIR ? Q : 1];
};

template <int Q, bool PAIR>
__device__ __forceinline__ void rotate_planes(const uint32_t (&W)[Q], Rot<Q, PAIR>& r)
{
#pragma unroll
    for (int p = 0; p < Q; ++p) r.A[p] = rotl(W[p], Q - 1 - p);
    if constexpr (PAIR) {
#pragma unroll
        for (int p = 0; p < Q; ++p) r.B[p] = rotl(W[p], 2 * Q - 5 - p);
    }
}

// One MFMA step's weights in three parts, so that a step's look-ups can be in
// flight while the previous step waits and multiplies: step_codes assembles
// the code register(s) of step P, step_lookup issues the LDS reads, step_pack
// forms the A fragment (8 x fp16, element e = column 8P + e of the word) once
// they have arrived.
struct StepCodes {
    // single tables: byte i of c0 / c1 = child code of column 8P + 2i / 8P + 2i + 1;
    // pair tables: byte i of c0 = code(8P + 2i) | code(8P + 2i + 1) << q, with
    // the LUT set of a two-set table above them (bit 2q); c1 unused
    uint32_t c0, c1;
};

struct StepRaw {
    uint32_t v[8];  // pair tables: v[0..3] = four fp16 pairs; single: v[0..7] = eight fp16 (low halves)
};

template <int Q, bool PAIR>
__device__ __forceinline__ StepCodes step_codes(const Rot<Q, PAIR>& r, int P, const RepMasks& M, uint32_t acc0)
{
    if constexpr (PAIR) {
        uint32_t acc = acc0;
#pragma unroll
        for (int p = 0; p < Q; ++p) {
            acc = and_or(r.A[p], M.m[rep_index(P + Q - 1 - p)], acc);
            acc = and_or(r.B[p], M.m[rep_index(P + 2 * Q - 1 - p)], acc);
        }
        return StepCodes{rotr(acc, P), 0u};
    } else {
        uint32_t c0 = 0, c1 = 0;
#pragma unroll
        for (int p = 0; p < Q; ++p) {
            c0 = and_or(r.A[p], M.m[rep_index(P + Q - 1 - p)], c0);
            c1 = and_or(r.A[p], M.m[rep_index(4 + P + Q - 1 - p)], c1);
        }
        return StepCodes{rotr(c0, P), rotr(c1, 4 + P)};
    }
}

template <bool PAIR>
__device__ __forceinline__ void step_lookup(const StepCodes& c, uint32_t lane_off, const char* lutb, StepRaw& raw)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (PAIR) {
            raw.v[i] = *(const uint32_t*)(lutb + lut_addr(c.c0, lane_off, i));
        } else {
            raw.v[2 * i] = *(const uint16_t*)(lutb + lut_addr(c.c0, lane_off, i));
            raw.v[2 * i + 1] = *(const uint16_t*)(lutb + lut_addr(c.c1, lane_off, i));
        }
    }
}

template <bool PAIR>
__device__ __forceinline__ half8_t step_pack(const StepRaw& raw)
{
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = PAIR ? raw.v[i] : (raw.v[2 * i] | (raw.v[2 * i + 1] << 16));
    return __builtin_bit_cast(half8_t, w);
}

// Form of rotate_planes / step_codes for a unit index P that differs
// between the lanes of a wave: rotating every plane word right by P as well
// turns the masks of unit P into those of unit 0, so the bit selects keep
// fixed (scalar) masks and the final rotate by P disappears; the rotate
// amounts are per lane (v_alignbit takes them from a register).  acc0 is the
// pair-table seed of unit 0.
template <int Q, bool PAIR>
__device__ __forceinline__ void rotate_planes_lane(const uint32_t (&W)[Q], int P, Rot<Q, PAIR>& r)
{
#pragma unroll
    for (int p = 0; p < Q; ++p) r.A[p] = rotr(W[p], P + p + 1 - Q);
    if constexpr (PAIR) {
#pragma unroll
        for (int p = 0; p < Q; ++p) r.B[p] = rotr(W[p], P + p + 5 - 2 * Q);
    }
}

template <int Q, bool PAIR>
__device__ __forceinline__ StepCodes step_codes_lane(const Rot<Q, PAIR>& r, uint32_t acc0)
{
    auto mask = [](int k) { return 0x01010101u << (k & 7); };
    if constexpr (PAIR) {
        uint32_t acc = acc0;
#pragma unroll
        for (int p = 0; p < Q; ++p) {
            acc = and_or(r.A[p], mask(Q - 1 - p), acc);
            acc = and_or(r.B[p], mask(2 * Q - 1 - p), acc);
        }
        return StepCodes{acc, 0u};
    } else {
        uint32_t c0 = 0, c1 = 0;
#pragma unroll
        for (int p = 0; p < Q; ++p) {
            c0 = and_or(r.A[p], mask(Q - 1 - p), c0);
            c1 = and_or(r.A[p], mask(4 + Q - 1 - p), c1);
        }
        return StepCodes{c0, rotr(c1, 4)};
    }
}

// LUT staging of a decode tile.  The block's LUT_q is stored in the slot
// layout [2^q][S] uint32 (slot j: entries of two rows in the low and high 16
// bits, see convert_lut); a tile of RG row groups owns NSLOT = 16 * RG
// consecutive slots from s0.  Single tables (q >= 5, and q = 4 with RG = 4):
// the tile's slots are copied to LDS as [entry][64 slots] (256-byte entry
// rows, RG = 2 tiles fill slots 0..31), so a look-up address is one v_perm of
// the code byte and the lane's byte offset 4 * slot + 2 * half.  Pair tables
// (RG = 2: q <= 4; RG = 4: q = 3; two weights per look-up) are built in LDS
// from the staged entries: entry a | b << q of a row holds LUT[a] |
// LUT[b] << 16.  RG = 2 keeps the row of half h of slot s at pair slot 32 h + s;
// RG = 4 keeps the slot and puts h above the pair code (a two-set q = 4 pair
// table would not fit).  Global reads are coalesced (a wave reads whole 128-
// or 256-byte runs of one entry) and LDS writes are 16 bytes per lane.  Split
// in two so callers can put other loads between the LUT loads and their first
// use: issue() starts every load of the wave, commit() writes LDS (pair
// tables: with a barrier between staging and building; the caller's barrier
// follows).
template <int Q, int RG, int NT = kThreads, bool WIDE = false>
struct LutLoad {
    static constexpr int NSLOT = 16 * RG;
    // WIDE (16- and 32-token passes): no q = 4 pair table for 64-row tiles, whose 64 KB
    // would leave no room for the wider activation slices
    static constexpr bool PAIR = RG == 2 ? Q <= (WIDE ? 3 : 4) : Q <= 3;
    static constexpr int NC = 1 << Q;
    static constexpr int PPE = NSLOT / 4;         // 16-byte pieces per entry
    static constexpr int BLOCKS = NC * PPE / 64;  // 64-piece blocks, one per wave load
    static constexpr int NW = NT / 64;
    static constexpr int PER = (BLOCKS + NW - 1) / NW;
    static_assert(NC * PPE % 64 == 0, "whole 64-piece blocks");
    u32x4 u[PER];

    __device__ __forceinline__ void issue(const uint32_t* lut, int S, int s0, int lane, int wave)
    {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int blk = wave + j * NW;  // wave-uniform
            if (blk < BLOCKS) {
                const int pc = blk * 64 + lane, e = pc / PPE, c = pc - e * PPE;
                u[j] = *(gu32x4p)(uintptr_t)(lut + (size_t)e * S + s0 + 4 * c);
            }
        }
    }

    __device__ __forceinline__ void commit(uint32_t* lds, uint32_t* stage, int lane, int wave)
    {
        uint32_t* dst = PAIR ? stage : lds;
        constexpr int STRIDE = PAIR ? NSLOT : 64;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int blk = wave + j * NW;
            if (blk < BLOCKS) {
                const int pc = blk * 64 + lane, e = pc / PPE, c = pc - e * PPE;
                *(u32x4*)(dst + e * STRIDE + 4 * c) = u[j];
            }
        }
        if constexpr (PAIR) {
            __syncthreads();
            constexpr int NPE = NC * NC;
            auto half16 = [](uint32_t v, int h) { return (v >> (16 * h)) & 0xffffu; };
            if constexpr (RG == 2) {
                for (int pe = wave; pe < NPE; pe += NW) {
                    const int h = lane >> 5, sl = lane & 31;
                    const int a = pe & (NC - 1), b = pe >> Q;
                    lds[(pe << 6) | lane] = half16(stage[a * NSLOT + sl], h) | (half16(stage[b * NSLOT + sl], h) << 16);
                }
            } else {
                for (int x = wave; x < 2 * NPE; x += NW) {
                    const int h = x / NPE, pe = x - h * NPE;
                    const int a = pe & (NC - 1), b = pe >> Q;
                    lds[(x << 6) | lane] = half16(stage[a * NSLOT + lane], h) | (half16(stage[b * NSLOT + lane], h) << 16);
                }
            }
        }
    }
};

// LDS byte offset of a look-up for the row held in half `h` of tile slot
// `sl` (pair tables: RG = 2 uses pair slot 32 h + sl, RG = 4 the slot with h
// carried in the code byte).
template <int Q, int RG, bool WIDE = false>
__device__ __forceinline__ uint32_t lut_lane_off(int sl, int h)
{
    if constexpr (LutLoad<Q, RG, kThreads, WIDE>::PAIR) return (uint32_t)(RG == 2 ? 32 * h + sl : sl) * 4u;
    return (uint32_t)sl * 4u + 2u * (uint32_t)h;
}

// A lane's row in a decode tile of RG 32-row groups (row group grp, lane row
// rho) and the LUT column that holds it.  gate_up tiles hold 16 * RG h-rows:
// groups [0, RG/2) are gate rows i, groups [RG/2, RG) the matching up rows
// I + i (LUT slot = h-row, gate in the low half, up in the high half).  down
// tiles hold 32 * RG consecutive rows (slot 32 m + r holds rows 64 m + r and
// 64 m + 32 + r).  Rows past the block are not valid: their loads use row 0
// and their outputs are never stored.
struct TileLane {
    int row, lrow;      // the row; the row the loads use
    bool valid;
    uint32_t lane_off;  // LDS byte offset of the row's LUT column
    bool set1;          // two-set pair tables: the row's table is the second set
};

template <int MODE, int Q, int RG, bool WIDE = false>
__device__ __forceinline__ TileLane tile_lane(int tile, int grp, int rho, int R)
{
    TileLane t;
    if (MODE == 0) {
        const int Iblk = R >> 1;
        const int sub = grp % (RG / 2), up = grp / (RG / 2);
        const int i = tile * (16 * RG) + 32 * sub + rho;
        t.valid = i < Iblk;
        t.row = up ? Iblk + i : i;
    } else {
        t.row = tile * (32 * RG) + 32 * grp + rho;
        t.valid = t.row < R;
    }
    t.lrow = t.valid ? t.row : 0;
    const int half = (MODE == 0 && RG == 4) ? grp / 2 : grp % 2;
    const int lslot = (MODE == 0 && RG == 4) ? 32 * (grp % 2) + rho : (RG == 4 ? 32 * (grp / 2) + rho : rho);
    t.lane_off = lut_lane_off<Q, RG, WIDE>(lslot, half);
    t.set1 = LutLoad<Q, RG, kThreads, WIDE>::PAIR && RG == 4 && half;
    return t;
}

// Code gather of one lane of a decode tile at width Q.  Single tables from
// q = 5 on take all eight code registers of a word by the bit transpose (4
// ops per swap: 96 per 128-column chunk against 146 for the and-or gather at
// q = 8); otherwise the planes are rotated once and each MFMA step gathers its
// own register (pair tables: two weights per look-up, the LUT set bit of a
// two-set table seeded above the 2q-bit pair code).  `zero` must be a zero the
// compiler cannot see through: with a literal zero it splits the bit-selects
// of the transpose's rows q..7 into more, cheaper ops.
template <int Q, int RG, bool WIDE = false>
struct WordDecoder {
    static constexpr bool PAIR = LutLoad<Q, RG, kThreads, WIDE>::PAIR;
    static constexpr bool TRANSPOSE = Q >= 5 && !PAIR;
    RepMasks masks;
    uint32_t zero;
    bool set1;
    Rot<Q, PAIR> rt;
    uint32_t X[8];

    __device__ __forceinline__ void prepare(const uint32_t (&W)[Q])
    {
        if constexpr (TRANSPOSE) transpose_codes<Q>(W, X, zero);
        else rotate_planes<Q, PAIR>(W, rt);
    }
    __device__ __forceinline__ StepCodes codes(int P) const
    {
        if constexpr (TRANSPOSE) return StepCodes{X[P], X[4 + P]};
        else return step_codes<Q, PAIR>(rt, P, masks, set1 ? rotl(0x01010101u << (2 * Q), P) : 0u);
    }
};

// ---------------------------------------------------------------- routing

// One wave per token: lane l holds the logits of experts l, l+64, l+128,
// l+192.  Each of the k rounds takes the wave-wide best entry by the order
// (value descending, expert index ascending) and retires it; the softmax runs
// over the k selected logits.  The order is one unsigned 64-bit key per entry:
// the logit's bits mapped so that unsigned order is numeric order (high word;
// -0 is folded into +0 first, so equal logits tie) above 0xffff - expert (low
// word); 0 marks a retired or absent entry.  Every step is a compare and two
// selects: no branches, no exec-mask changes.
struct RouteKey {
    uint32_t hi, lo;
};

__device__ __forceinline__ RouteKey route_key(float v, int e)
{
    const uint32_t u = __float_as_uint(v + 0.0f);  // -0 + 0 = +0
    return RouteKey{(u & 0x80000000u) ? ~u : (u | 0x80000000u), 0xffffu - (uint32_t)e};
}

__device__ __forceinline__ float route_key_value(uint32_t hi)
{
    return __uint_as_float((hi & 0x80000000u) ? (hi & 0x7fffffffu) : ~hi);
}

__device__ __forceinline__ void route_key_max(RouteKey& a, uint32_t bh, uint32_t bl)
{
    const uint64_t ka = ((uint64_t)a.hi << 32) | a.lo, kb = ((uint64_t)bh << 32) | bl;
    const bool take = kb > ka;
    a.hi = take ? bh : a.hi;
    a.lo = take ? bl : a.lo;
}

// One DPP step of the wave-wide maximum: lanes take the key the pattern
// brings in if it is larger; lanes whose row is masked off keep their own.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void route_dpp_step(RouteKey& a)
{
    const uint32_t oh = (uint32_t)__builtin_amdgcn_update_dpp((int)a.hi, (int)a.hi, CTRL, ROW_MASK, 0xf, false);
    const uint32_t ol = (uint32_t)__builtin_amdgcn_update_dpp((int)a.lo, (int)a.lo, CTRL, ROW_MASK, 0xf, false);
    route_key_max(a, oh, ol);
}

// Wave-wide maximum of an unsigned word (the same DPP pattern as the key
// maximum below; 0 is the identity, so lanes a step leaves out keep theirs).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));  // row_half_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));  // row_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Top-k of token t's logits for E <= 64, lane = expert: each pick is the
// wave maximum of the 32-bit high key words of the experts still in play,
// then the lowest lane holding it (the same order as the 64-bit keys: value
// descending, index ascending), so the results equal route_token's with a
// quarter of its instructions on the dependent chain.
__device__ __forceinline__ int route_token64(const float* __restrict__ logits, int t, int E, int k, float& wout)
{
    const int lane = threadIdx.x & 63;
    const uint32_t hi = route_key(logits[(size_t)t * E + min(lane, E - 1)], lane).hi;
    bool alive = lane < E;
    int out = -1;
    float mine = 0.0f, m = 0.0f, s = 0.0f;
#pragma unroll 1
    for (int j = 0; j < k; ++j) {
        const uint32_t mx = wave_max_u32(alive ? hi : 0u);
        const uint64_t win = __ballot(alive && hi == mx);
        const int w = __ffsll((long long)win) - 1;
        alive = alive && lane != w;
        const float bv = route_key_value(mx);
        if (j == 0) m = bv;
        const float ex = expf(bv - m);
        s += ex;
        const bool me = lane == j;
        out = me ? w : out;
        mine = me ? ex : mine;
    }
    wout = lane < k ? mine / s : 0.0f;
    return out;
}

// Top-k of token t's logits by one wave; lanes j < k hold the j-th expert
// and its gate weight (returned; other lanes return -1).
__device__ __forceinline__ int route_token(const float* __restrict__ logits, int t, int E, int k, float& wout)
{
    if (E <= 64) return route_token64(logits, t, E, k, wout);
    const int lane = threadIdx.x & 63;
    const float* l = logits + (size_t)t * E;
    RouteKey key[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        const float v = l[min(e, E - 1)];  // in bounds on every lane; absent entries drop below
        const RouteKey kk = route_key(v, e);
        key[i] = e < E ? kk : RouteKey{0u, 0u};
    }
    // pick j is kept by lane j; the softmax sums exp(pick - best) in pick
    // order (a rolled loop keeps the code small: every routing workgroup
    // runs it once)
    int out = -1;
    float mine = 0.0f, m = 0.0f, s = 0.0f;
#pragma unroll 1
    for (int j = 0; j < k; ++j) {
        RouteKey b = key[0];
#pragma unroll
        for (int i = 1; i < 4; ++i) route_key_max(b, key[i].hi, key[i].lo);
        // wave-wide maximum by DPP steps (no LDS round trips): pairs and
        // quads, mirrored halves of 8, mirrored rows of 16, then rows 0 / 2
        // into 1 / 3 and row 1 into 2 / 3; lane 63 ends with the maximum
        route_dpp_step<0xB1, 0xf>(b);   // quad_perm [1,0,3,2]
        route_dpp_step<0x4E, 0xf>(b);   // quad_perm [2,3,0,1]
        route_dpp_step<0x141, 0xf>(b);  // row_half_mirror
        route_dpp_step<0x140, 0xf>(b);  // row_mirror
        route_dpp_step<0x142, 0xa>(b);  // row_bcast:15
        route_dpp_step<0x143, 0xc>(b);  // row_bcast:31
        const uint32_t wh = (uint32_t)__builtin_amdgcn_readlane((int)b.hi, 63);
        const uint32_t wl = (uint32_t)__builtin_amdgcn_readlane((int)b.lo, 63);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool hit = key[i].lo == wl;
            key[i].hi = hit ? 0u : key[i].hi;
            key[i].lo = hit ? 0u : key[i].lo;
        }
        const float bv = route_key_value(wh);
        if (j == 0) m = bv;
        const float ex = expf(bv - m);
        s += ex;
        const bool me = lane == j;
        out = me ? (int)(0xffffu - wl) : out;
        mine = me ? ex : mine;
    }
    wout = lane < k ? mine / s : 0.0f;
    return out;
}

// One token's picks in the form the callers store: lane j < k holds pick j.
struct RoutePick {
    int j;    // pick index 0..k-1, or -1 on lanes >= k
    int e;    // the picked expert
    float w;  // its gate weight
};

__device__ __forceinline__ RoutePick route_pick(const float* __restrict__ logits, int t, int E, int k)
{
    float wv;
    const int e = route_token(logits, t, E, k, wv);
    const int lane = threadIdx.x & 63;
    return RoutePick{lane < k ? lane : -1, e, wv};
}

// Top-k of token t's logits by one lane, for E <= EM (8, 16 or 32): the
// same keys, picks and softmax arithmetic as route_token (so the results are
// bit-identical), with the E keys in the lane's registers instead of across a
// wave.  A wave routes 64 tokens at once; a batch of up to 1024 tokens takes
// one round trip for its logits instead of one per token and wave.
template <int EM>
__device__ __forceinline__ void route_lane(const float* __restrict__ logits, int t, int E, int k, int (&eo)[8],
                                           float (&wo)[8])
{
    // the high key words only: an entry's low word is fixed by its index, so
    // the order (value descending, index ascending) is a scan in index order
    // that replaces the best on a strictly larger value; picked entries are
    // masked out by a bit each
    const float* l = logits + (size_t)t * E;
    uint32_t hi[EM];
#pragma unroll
    for (int e = 0; e < EM; ++e) hi[e] = route_key(l[min(e, E - 1)], e).hi;
    uint32_t used = 0;
    float m = 0.0f, s = 0.0f, ex[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        ex[j] = 0.0f;
        eo[j] = -1;
        if (j < k) {
            uint32_t bh = 0u;
            int be = -1;
#pragma unroll
            for (int e = 0; e < EM; ++e) {
                const bool take = e < E && !((used >> e) & 1u) && (be < 0 || hi[e] > bh);
                bh = take ? hi[e] : bh;
                be = take ? e : be;
            }
            used |= 1u << be;
            const float bv = route_key_value(bh);
            if (j == 0) m = bv;
            ex[j] = expf(bv - m);
            s += ex[j];
            eo[j] = be;
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) wo[j] = j < k ? ex[j] / s : 0.0f;
}

// Largest expert count routed one token per lane.
constexpr int kLaneRouteMaxE = 32;

__device__ __forceinline__ void route_lane_any(const float* __restrict__ logits, int t, int E, int k, int (&eo)[8],
                                               float (&wo)[8])
{
    if (E <= 8) route_lane<8>(logits, t, E, k, eo, wo);
    else if (E <= 16) route_lane<16>(logits, t, E, k, eo, wo);
    else route_lane<32>(logits, t, E, k, eo, wo);
}

__global__ void __launch_bounds__(256) route_topk_lane_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                              int32_t* __restrict__ idx, float* __restrict__ w)
{
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= T) return;
    int eo[8];
    float wo[8];
    route_lane_any(logits, t, E, k, eo, wo);
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (j < k) {
            idx[(size_t)t * k + j] = eo[j];
            w[(size_t)t * k + j] = wo[j];
        }
}

__global__ void __launch_bounds__(256) route_topk_kernel(const float* __restrict__ logits, int T, int E,
                                                         int k, int32_t* __restrict__ idx,
                                                         float* __restrict__ w)
{
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // whole wave
    const RoutePick p = route_pick(logits, t, E, k);
    if (p.j >= 0) {
        idx[(size_t)t * k + p.j] = p.e;
        w[(size_t)t * k + p.j] = p.w;
    }
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts (no LDS round trips): shifts 1, 2, 4, 8 inside each 16-lane
// row, then lane 15 of rows 0 / 2 into rows 1 / 3, then lane 31 into rows 2
// and 3.  Lanes whose DPP source is outside the row, or whose row is masked
// off, add 0.
__device__ __forceinline__ int wave_inclusive_sum(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

// Stable counting sort of the n assignments by expert (one 1024-thread
// workgroup); idx may point to global memory or LDS.
__device__ __forceinline__ void permute_body(const int32_t* idx, int n, int E, int32_t* __restrict__ offsets,
                                             int32_t* __restrict__ sorted, int* cnt, int* base, int (*wcnt)[256])
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int e = tid; e < E; e += 1024) cnt[e] = 0;
    __syncthreads();
    for (int a = tid; a < n; a += 1024) {
        const int e = idx[a];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    if (wave == 0) {  // exclusive scan of the counts: 4 experts per lane + a wave scan
        int c[4], s = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane * 4 + i;
            c[i] = e < E ? cnt[e] : 0;
            s += c[i];
        }
        const int incl = wave_inclusive_sum(s);
        int ex = incl - s;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane * 4 + i;
            if (e < E) {
                base[e] = ex;
                offsets[e] = ex;
            }
            ex += c[i];
        }
        if (lane == 63) offsets[E] = incl;
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

__global__ void __launch_bounds__(1024) permute_kernel(const int32_t* __restrict__ idx, int n, int E,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ sorted)
{
    __shared__ int cnt[256];
    __shared__ int base[256];
    __shared__ int wcnt[16][256];
    permute_body(idx, n, E, offsets, sorted, cnt, base, wcnt);
}

// Stable counting sort of n <= 64 assignments by wave 0 alone, one
// assignment per lane (LDS operations of one wave complete in order, so no
// barrier is needed).  sidx, cnt and base are LDS; offsets and sorted may be
// global memory or LDS.
__device__ __forceinline__ void sort_small(const int* sidx, int n, int E, int32_t* offsets, int32_t* sorted,
                                           int* cnt, int* base)
{
    const int lane = threadIdx.x & 63;
    int e = lane < n ? sidx[lane] : 511;
    if (e < 0 || e >= E) e = 511;
    for (int x = lane; x < E; x += 64) cnt[x] = 0;
    if (e < E) atomicAdd(&cnt[e], 1);
    int c[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int x = lane * 4 + i;
        c[i] = x < E ? cnt[x] : 0;
        sum += c[i];
    }
    const int incl = wave_inclusive_sum(sum);
    int ex = incl - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int x = lane * 4 + i;
        if (x < E) {
            base[x] = ex;
            offsets[x] = ex;
        }
        ex += c[i];
    }
    if (lane == 63) offsets[E] = incl;
    // rank among the lanes with the same expert (lanes = assignments in order)
    unsigned long long m = ~0ull;
#pragma unroll
    for (int b = 0; b < 9; ++b) {
        const int bit = (e >> b) & 1;
        const unsigned long long bal = __ballot(bit);
        m &= bit ? bal : ~bal;
    }
    const int rank = __popcll(m & ((1ull << lane) - 1ull));
    if (e < E) sorted[base[e] + rank] = lane;
}

// Routing and permutation of a decode-sized batch in one workgroup: the
// threads route the tokens (up to 32 experts one token per lane, else one
// token per wave at a time), the assignments stay in LDS, and the same
// workgroup sorts them.  Results equal those of the two separate kernels.
__global__ void __launch_bounds__(1024) route_permute_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                             int32_t* __restrict__ idx, float* __restrict__ w,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ sorted)
{
    __shared__ int cnt[256];
    __shared__ int base[256];
    __shared__ int wcnt[16][256];
    __shared__ int sidx[kFusedMaxAssign];
    const int wave = threadIdx.x >> 6;
    if (E <= kLaneRouteMaxE) {
        for (int t = threadIdx.x; t < T; t += 1024) {
            int eo[8];
            float wo[8];
            route_lane_any(logits, t, E, k, eo, wo);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (j < k) {
                    idx[(size_t)t * k + j] = eo[j];
                    w[(size_t)t * k + j] = wo[j];
                    sidx[t * k + j] = eo[j];
                }
        }
    } else {
        for (int t = wave; t < T; t += 16) {
            const RoutePick p = route_pick(logits, t, E, k);
            if (p.j >= 0) {
                idx[(size_t)t * k + p.j] = p.e;
                w[(size_t)t * k + p.j] = p.w;
                sidx[t * k + p.j] = p.e;
            }
        }
    }
    __syncthreads();
    const int n = T * k;
    if (n > 64) {
        permute_body(sidx, n, E, offsets, sorted, cnt, base, wcnt);
        return;
    }
    // up to 64 assignments: wave 0 alone (see sort_small)
    if (wave != 0) return;
    sort_small(sidx, n, E, offsets, sorted, cnt, base);
}

// ---------------------------------------------------------------- FFN GEMV

// Contraction of one 64-row tile on the matrix cores (v_mfma_f32_32x32x16_f16).
//
// MODE 0: gate_up. Row group 0 = 32 gate rows, row group 1 = the matching 32
//         up rows; input x (fp16); epilogue h = silu(g) * u rounded to fp16
//         (the MFMA operand of down; accumulation stays fp32).
// MODE 1: down. Row groups 0 / 1 = 64 consecutive output rows; input h
//         (fp16); the K range may be split over several workgroups, each
//         writing the fp32 partial expert output of its split (summed in
//         split order by the combine).
//
// Waves 0-3 own row group 0 and waves 4-7 row group 1; the four waves of a
// group split K by 128-column chunks.  Lane l = (rho = l % 32, kh = l / 32)
// decodes row rho of its group and, in each chunk, words 2*kh and 2*kh + 1
// (8-byte loads: a wave reads 32 rows x 16 B = 512 B contiguous per plane).
// Word pair u pairs word u (kh = 0) with word 2 + u (kh = 1) in one 16-deep
// MFMA step set: step P takes columns 8P..8P+7 of each word, which is exactly
// what the gather produces for register P.  The tokens of a pass (up to 8)
// are the MFMA's N columns; a weight is decoded once per pass.
//
// Memory pipeline.  Each wave keeps D chunks of plane loads in flight (a
// static ring, so no in-flight register is ever moved) and loads the next
// chunk's activations one chunk ahead: the 64 lanes fetch the pass's tokens x
// 128 columns cooperatively (16 bytes each) and store them in the wave's own
// LDS slice, from which the B fragments are read.  B reads therefore count on
// lgkmcnt only, and waiting for this chunk's data never waits for the
// prefetch of later chunks (global loads complete in order on vmcnt).  The
// partials of a group's four waves are summed in wave order through the slice
// region after the pass; the LUT stays resident for every pass.
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const u32x2* gu32x2p;
typedef __attribute__((address_space(1))) const u32x4* gcu32x4p;
typedef __attribute__((address_space(4))) const int32_t* ci32p;

constexpr int kTokPass = 8;               // most tokens per pass
constexpr int kSliceWords = 512;          // per-wave slice: 8 rows x 16 units of 16 B
static_assert(kWaves * kSliceWords >= kStageWords, "pair staging lives in the slice region");
static_assert(kWaves * 32 * kTokPass <= kWaves * kSliceWords, "reduction lives in the slice region");

// The kernel's FfnArgs viewed in the (constant) kernarg segment: fields are
// read with scalar loads on demand instead of being copied to scratch.
typedef __attribute__((address_space(4))) const FfnArgs KArgs;
__device__ __forceinline__ KArgs& kernel_args()
{
    return *(KArgs*)__builtin_amdgcn_kernarg_segment_ptr();
}

// Words 2*kh, 2*kh+1 of chunk c of `row` from each of the q planes.  Plane
// pointers are read from the page-table entry (scalar loads, K-cache hits).
// The loads are unconditional (callers pass an in-range row even for lanes
// whose row is past the block; those lanes' outputs are never stored): a
// lane-divergent load makes the compiler wait for every outstanding load
// (vmcnt(0)), which would serialise the prefetch ring.  KEEP: ordinary loads
// instead of nontemporal ones, for launches whose tiles are streamed more
// than once (more than one pass of tokens), so the later passes can hit the
// MALL.
template <int Q, bool KEEP = false>
__device__ __forceinline__ void load_pair_words(u32x2 (&pg)[Q], const BlockDesc* __restrict__ bd, int c, int R,
                                                int row, int kh)
{
    // byte offset in 32 bits (a plane is below 4 GB): the loads take the
    // plane pointer as a scalar base and one shared vector offset
    const uint32_t at = (((uint32_t)c * (uint32_t)R + (uint32_t)row) * 2u + (uint32_t)kh) * 8u;
    const __attribute__((address_space(4))) BlockDesc* cbd = (const __attribute__((address_space(4))) BlockDesc*)(uintptr_t)bd;
#pragma unroll
    for (int p = 0; p < Q; ++p) {
        if constexpr (KEEP) pg[p] = *((gu32x2p)((uintptr_t)cbd->planes[p] + at));
        else pg[p] = __builtin_nontemporal_load((gu32x2p)((uintptr_t)cbd->planes[p] + at));
    }
}

// 16-byte unit g (8 fp16 columns) of row j of a slice: the rows are the
// pass's tokens (x for gate_up, h for down).  The unit index is XOR-swizzled
// with the token (its low four bits) so the B reads of different tokens in
// one instruction fall in different banks.
__device__ __forceinline__ int slice_unit(int j, int t, int g)
{
    return j * 16 + (g ^ (t & 15));
}

// FUSED (gate_up of a launch that routed the batch itself): lane i of tokreg
// holds the slot's i-th sorted assignment instead of a.sorted in memory.
template <int MODE, int Q, int RG, bool FUSED = false, bool KEEP = false, int TP = 8>
__device__ __forceinline__ void mfma_block(const KArgs& a, const BlockDesc* __restrict__ bd, bool shared, int p0,
                                           int ntok, int tile, int split, int nsplit, uint32_t* lds, int tokreg = 0)
{
    // TP tokens per pass: 8, or 16 / 32 (WIDE) for launches where experts hold
    // more than 8 / 16 tokens, so each weight is decoded once per 16 / 32
    // tokens (the MFMA's B operand has 32 token columns in every case).
    // SHARE (32-token passes): the RG waves of a K range (one per row group)
    // share one 8 KB activation slice, each loading 32 / RG of the 32 token
    // rows, with a workgroup barrier before and after each chunk's slice
    // store; this keeps the registers of 8- or 16-token passes.  64-row tiles
    // keep their four slices in LUT space the tile does not use, 128-row
    // tiles their two in the slice region after the LUT.
    constexpr bool WIDE = TP >= 16;
    constexpr bool SHARE = TP == 32;
    static_assert(TP == 8 || (TP == 16 && RG == 2 && !FUSED) || (TP == 32 && !FUSED),
                  "16-token passes: 64-row tiles; 16- and 32-token passes: routing outside");
    constexpr int D = Q <= 4 ? 2 : 1;      // chunks of plane loads in flight
    constexpr int NLOAD = SHARE ? 32 / RG : TP;  // token rows this wave loads per chunk
    constexpr int NPART = NLOAD / 4;       // activation loads per lane and chunk
    constexpr int SB = TP * 256;           // bytes of a slice (TP token rows x 256 B)
    constexpr int KW = kWaves / RG;        // waves per row group (K split)
    constexpr bool PAIR = LutLoad<Q, RG, kThreads, WIDE>::PAIR;
    constexpr int HR = 16 * RG;            // gate_up: h rows per tile (gate and up rows each)
    constexpr int TR = 32 * RG;            // down: output rows per tile
    const int tid = threadIdx.x, lane = tid & 63, rho = lane & 31, kh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave / KW, kw = wave % KW;
    const int R = bd->R;
    const int nchunks = bd->nchunks, kwords = bd->kwords;
    const int K = kwords * 32;
    const int Iblk = R >> 1;
    const TileLane tl = tile_lane<MODE, Q, RG, WIDE>(tile, grp, rho, R);
    const int lrow = tl.lrow;  // in-range load row
    const int cps = (nchunks + nsplit - 1) / nsplit;
    const int c_begin = split * cps;
    const int c_end = min(nchunks, c_begin + cps);
    const int first = c_begin + kw;
    const int nch = first < c_end ? (c_end - first + KW - 1) / KW : 0;
    // chunk iterations: SHARE runs the same count in every wave (the barriers
    // of the shared slices), the waves past their own chunks on padding chunks
    const int nloop = SHARE ? (c_end - c_begin + KW - 1) / KW : nch;
    const int lastc = nch > 0 ? first + (nch - 1) * KW : 0;  // chunk 0 always exists
    const int TK = a.T * a.k;

    // byte b of activation slice w (TP token rows x 16 units of 16 B).
    // 8-token passes: 2 KB per wave after the LUT.  16-token passes (64-row
    // tiles): 4 KB per wave, 32-token passes: 8 KB per pair of waves, inside
    // the 64 KB LUT area in space the tile's table never uses: the upper half
    // of every 256-byte entry row at q = 8 (a 64-row tile fills slots 0..31),
    // else rows 128..255 (2^q <= 128 single entries, or 64 rows of the q = 3
    // pair table).
    char* const ldsb = (char*)lds;
    // Double-buffered shared slices (one barrier per chunk: a chunk's store
    // goes to the buffer every wave finished reading before the previous
    // chunk's barrier): 128-row tiles below q = 8 keep both buffers' two
    // slices in LUT rows 128..255 (a table of <= 128 entries leaves them
    // free); 64-row tiles up to q = 6 keep buffer 0's four slices in rows
    // 128..255 and buffer 1's in the slice region after the LUT (slices 0, 1)
    // and rows 64..127 (slices 2, 3; tables of <= 64 entries).  The others
    // keep one buffer and a second barrier.
    constexpr bool DBUF4 = SHARE && RG == 4 && Q < 8;
    constexpr bool DBUF2 = SHARE && RG == 2 && Q <= 6;
    constexpr bool DBUF = DBUF4 || DBUF2;
    int sbuf = 0;  // DBUF: this chunk's buffer
    auto slice_at = [&](int w, int b) -> char* {
        if constexpr (DBUF4) return ldsb + 32768 + (2 * sbuf + w) * SB + b;
        else if constexpr (DBUF2) {
            if (sbuf == 0) return ldsb + 32768 + w * SB + b;
            return w < 2 ? ldsb + kLutBytes + w * SB + b : ldsb + 16384 + (w - 2) * SB + b;
        } else if constexpr (SHARE && RG == 4) return ldsb + kLutBytes + w * SB + b;
        else if constexpr (!WIDE) return ldsb + kLutBytes + w * (kSliceWords * 4) + b;
        else if constexpr (Q == 8) return ldsb + (((((SB / 128) * w + (b >> 7)) << 8) | 128) | (b & 127));
        else return ldsb + 32768 + w * SB + b;
    };
    const int sl = SHARE ? kw : wave;  // this wave's activation slice
    const int tb = SHARE ? (32 / RG) * grp : 0;  // first slice row this wave loads
    const uint32_t lane_off = tl.lane_off;
    const char* lutb = (const char*)lds;
    WordDecoder<Q, RG, WIDE> dec;
    dec.masks = make_masks();
    // a zero the compiler cannot prove (T >= 1 here)
    dec.zero = (uint32_t)__builtin_amdgcn_readfirstlane(a.T >> 30);
    dec.set1 = tl.set1;

    // cooperative activation loads: lane = (token xt, 16-byte unit xg)
    const int xt = lane >> 4, xg = lane & 15;

    u32x2 pg[D][Q];
    u32x4 xv[NPART];
    const uint16_t* xsrc[NPART];
    int nt = 0;

    // Activation rows of the pass starting at t0: tokens tb + xt + 4 pp (x
    // for gate_up, h for down; tokens past the pass repeat its last token,
    // whose slots are never read).
    auto set_sources = [&](int t0) {
        nt = min(TP, ntok - t0);
        if (MODE == 0) {
            int tok[NPART];
            if (shared) {
#pragma unroll
                for (int pp = 0; pp < NPART; ++pp) tok[pp] = t0 + min(tb + xt + 4 * pp, nt - 1);
            } else {
                int sa[NLOAD];
                if constexpr (FUSED) {
#pragma unroll
                    for (int j = 0; j < NLOAD; ++j) sa[j] = __builtin_amdgcn_readlane(tokreg, t0 + min(j, nt - 1));
                } else {
                    // the pass's assignment ids through scalar loads (lgkmcnt)
                    const ci32p srt = (ci32p)(uintptr_t)a.sorted;
                    const int base = p0 + t0;
#pragma unroll
                    for (int j = 0; j < NLOAD; ++j) sa[j] = srt[base + min(tb + j, nt - 1)];
                }
#pragma unroll
                for (int h = 0; h < NPART; ++h) {
                    const int te = xt + 4 * h;
                    int v = sa[0];
#pragma unroll
                    for (int j = 1; j < NLOAD; ++j) v = te == j ? sa[j] : v;
                    tok[h] = v / a.k;
                }
            }
#pragma unroll
            for (int pp = 0; pp < NPART; ++pp) xsrc[pp] = a.x + (size_t)tok[pp] * a.H;
        } else {
#pragma unroll
            for (int h = 0; h < NPART; ++h) {
                const int te = min(tb + xt + 4 * h, nt - 1);
                const int hrow = shared ? TK + t0 + te : p0 + t0 + te;
                xsrc[h] = a.h + (size_t)hrow * a.hstride;
            }
        }
    };
    // activation unit of chunk c (column clamped into the row; the store zeroes it)
    auto issue_x = [&](int c) {
        const int col = min(c * kChunkCols + 8 * xg, K - 8);
#pragma unroll
        for (int pp = 0; pp < NPART; ++pp) xv[pp] = *(gcu32x4p)(uintptr_t)(xsrc[pp] + col);
    };
    auto issue_ring = [&]() {
        issue_x(first);
#pragma unroll
        for (int d = 0; d < D; ++d) load_pair_words<Q, KEEP>(pg[d], bd, min(first + d * KW, lastc), R, lrow, kh);
    };

    // pass 0: LUT loads first, then the ring's first loads, then LUT -> LDS
    {
        LutLoad<Q, RG, kThreads, WIDE> ls;
        ls.issue(bd->lut, bd->slots, tile * LutLoad<Q, RG, kThreads, WIDE>::NSLOT, lane, wave);
        set_sources(0);
        if (ntok > 0) issue_ring();
        ls.commit(lds, lds + kLutBytes / 4, lane, wave);
        __syncthreads();
    }

    for (int t0 = 0; t0 < ntok; t0 += TP) {
        if (t0 > 0) {
            set_sources(t0);
            issue_ring();
        }
        const int te = rho < nt ? rho : 0;  // B lanes past the pass read token 0
        const bool nvalid = rho < nt;
        f32x16 C = {};

        for (int ci0 = 0; ci0 < nloop; ci0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                // keep the scheduler from hoisting the next slot's work (which
                // would wait on that slot's loads too)
                __builtin_amdgcn_sched_barrier(0);
                const int ci = ci0 + d;
                // Waves w and w + 4 share a SIMD, and issue arbitration favours
                // the older one: waves 4-7 (gate_up's up rows) ended their K loop
                // ~3 us after waves 0-3.  Swapping which wave of the pair has the
                // higher issue priority every chunk keeps the pair in step
                // (Qwen-shaped batch 4 step 0.0373 -> 0.0362 ms).
                if constexpr (!SHARE) {
                    if ((ci ^ (wave >> 2)) & 1) __builtin_amdgcn_s_setprio(1);
                    else __builtin_amdgcn_s_setprio(0);
                }
                const bool live = ci < nch;  // padding chunk of the ring: B = 0
                const int c = min(first + ci * KW, lastc);
                // this chunk's activations -> the wave's slice (zero past K and
                // in padding chunks)
                const bool ok = live && c * kChunkCols + 8 * xg < K;
                if constexpr (DBUF) sbuf = ci & 1;
                if constexpr (SHARE && !DBUF) __syncthreads();  // the partner waves have read the slice's last chunk
#pragma unroll
                for (int pp = 0; pp < NPART; ++pp) {
                    const int j = tb + 4 * pp + xt;
                    *(u32x4*)slice_at(sl, 16 * slice_unit(j, j, xg)) = ok ? xv[pp] : u32x4{0, 0, 0, 0};
                }
                if constexpr (SHARE) __syncthreads();  // every part of this chunk's tokens is in the slice
                // prefetch: next chunk's activations, then the planes D chunks on
                u32x2 cur[Q];
#pragma unroll
                for (int p = 0; p < Q; ++p) cur[p] = pg[d][p];
                issue_x(min(c + KW, lastc));
                load_pair_words<Q, KEEP>(pg[d], bd, min(c + D * KW, lastc), R, lrow, kh);
                // the 8 MFMA steps s = 4u + P of the chunk (word pair u,
                // columns 8P..8P+7), pipelined by one step: the B read and the
                // LUT look-ups of step s + 1 are issued before step s's MFMA
                // finishes, and step s + 1's code gather runs while step s's
                // reads are in flight.
                auto b_unit = [&](int s, int row) { return slice_unit(row, te, 4 * (2 * kh + (s >> 2)) + (s & 3)); };
                auto prepare = [&](int u) {
                    uint32_t W[Q];
#pragma unroll
                    for (int p = 0; p < Q; ++p) W[p] = cur[p][u];
                    dec.prepare(W);
                };
                auto codes = [&](int P) { return dec.codes(P); };
                auto b_read = [&](int s) { return *(const u32x4*)slice_at(sl, 16 * b_unit(s, te)); };
                prepare(0);
                u32x4 bh = b_read(0);
                StepRaw raw;
                step_lookup<PAIR>(codes(0), lane_off, lutb, raw);
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    StepCodes next{0u, 0u};
                    if (s < 7 && s != 3) next = codes((s + 1) & 3);
                    const half8 A = step_pack<PAIR>(raw);
                    C = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, __builtin_bit_cast(half8, bh), C, 0, 0, 0);
                    if (s == 3) {  // word pair 1, once step 3's operands are consumed
                        prepare(1);
                        next = codes(0);
                    }
                    if (s < 7) {
                        bh = b_read(s + 1);
                        step_lookup<PAIR>(next, lane_off, lutb, raw);
                    }
                }
            }
        }

        if constexpr (!SHARE) __builtin_amdgcn_s_setprio(0);
        // cross-wave reduction through the slices: wave w's partial of (row r,
        // token n) at word rix(r, n) = 32 n + (r ^ n) of its slice (SHARE: of
        // half w % 2 of slice w / 2), token-major so the epilogue reads and
        // stores run along rows; the XOR keeps both the partial stores (lanes
        // = tokens) and the epilogue reads (lanes = rows) free of bank
        // conflicts.  SHARE with 128-row tiles sums in two phases in the 16 KB
        // slice region (row group g's sums at 4 KB g): the partials of K-wave
        // 1, then K-wave 0 adds its own (the same order and rounding as the
        // one-phase sum 0 + p0 + p1).
        static_assert(!(SHARE && RG == 4) || KW == 2, "two-phase sum of two K-waves");
        sbuf = 0;  // the 64-row tiles' reduction uses buffer 0's contiguous 32 KB
        auto rix = [](int r, int n) { return 32 * n + (r ^ (n & 31)); };
        auto red4 = [&](int g, int r, int n) -> float* { return (float*)(ldsb + kLutBytes + 4096 * g + 4 * rix(r, n)); };
        __syncthreads();
        auto red = [&](int w, int r, int n) -> float* {
            if constexpr (SHARE) return (float*)slice_at(w >> 1, 4096 * (w & 1) + 4 * rix(r, n));
            else return (float*)slice_at(w, 4 * rix(r, n));
        };
        // this lane's partial C[i] (row r_i = 8 (i / 4) + 4 kh + i % 4, token
        // rho) goes to word 32 rho + (r_i ^ rho) = 32 rho + (c_i ^ mx); mx is
        // made opaque here so the sixteen addresses are formed per pass and not
        // hoisted into registers held across the K loop
        int mx = (kh << 2) ^ rho;
        asm volatile("" : "+v"(mx));
        auto wix = [&](int i) { return 32 * rho + ((((i >> 2) << 3) | (i & 3)) ^ mx); };
        if constexpr (SHARE && RG == 4) {
            if (nvalid && kw == 1) {
#pragma unroll
                for (int i = 0; i < 16; ++i) *(float*)(ldsb + kLutBytes + 4096 * grp + 4 * wix(i)) = C[i];
            }
            __syncthreads();
            if (nvalid && kw == 0) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float* p = (float*)(ldsb + kLutBytes + 4096 * grp + 4 * wix(i));
                    *p = C[i] + *p;
                }
            }
        } else if (nvalid) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if constexpr (SHARE) *(float*)slice_at(wave >> 1, 4096 * (wave & 1) + 4 * wix(i)) = C[i];
                else *(float*)slice_at(wave, 4 * wix(i)) = C[i];
            }
        }
        __syncthreads();
        if (MODE == 0) {
            // rows fastest: a wave stores 64 consecutive h entries of one token
            for (int idx = tid; idx < HR * nt; idx += kThreads) {
                const int n = idx / HR, hr = idx % HR;
                const int sub = hr >> 5, r = hr & 31;
                float g = 0.0f, u = 0.0f;
                if constexpr (SHARE && RG == 4) {
                    g = *red4(sub, r, n);
                    u = *red4(RG / 2 + sub, r, n);
                } else {
#pragma unroll
                    for (int w = 0; w < KW; ++w) {
                        g += *red(sub * KW + w, r, n);
                        u += *red((RG / 2 + sub) * KW + w, r, n);
                    }
                }
                const int i = tile * HR + hr;
                if (i < Iblk) {
                    const float h = g / (1.0f + __expf(-g)) * u;
                    const int hrow = shared ? TK + t0 + n : p0 + t0 + n;
                    a.h[(size_t)hrow * a.hstride + i] = __builtin_bit_cast(uint16_t, (_Float16)h);
                }
            }
        } else {
            for (int idx = tid; idx < TR * nt; idx += kThreads) {
                const int n = idx / TR, rt = idx % TR;
                const int g = rt >> 5, r = rt & 31;
                float d = 0.0f;
                if constexpr (SHARE && RG == 4) {
                    d = *red4(g, r, n);
                } else {
#pragma unroll
                    for (int w = 0; w < KW; ++w) d += *red(g * KW + w, r, n);
                }
                const int orow_r = tile * TR + rt;
                if (orow_r < R) {
                    const int orow = shared ? TK + t0 + n : a.sorted[p0 + t0 + n];
                    a.dout[((size_t)split * a.drows + orow) * a.H + orow_r] = d;
                }
            }
        }
        __syncthreads();
    }
}

// The expert of routed slot `slot`: the active experts (at least one routed
// assignment) ordered by committed width, widest first, then by index, so the
// largest blocks are dispatched first and the last workgroups of a launch are
// the cheapest.  Every lane tests up to four experts (offsets and widths are
// loaded together: one memory round trip), ballots give the bitmap of active
// experts of each width, and the lane holding the wanted expert is found by its
// rank; its offsets are read from that lane.  Wave-uniform result, e = -1 if
// the slot has no expert.
struct SlotExpert {
    int e, p0, ntok;
};

// Committed widths of the E blocks of one module, experts lane + 64 g.
__device__ __forceinline__ void load_widths(const BlockDesc* __restrict__ table, int module, int E, int (&q)[4])
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int e = 64 * g + lane;
        q[g] = table[(e < E ? e : 0) * 2 + module].q;  // in-range address for every lane
    }
}

// Expert of a routed slot: the active experts (offsets[e + 1] > offsets[e])
// ordered by decreasing width, then by index.  offsets may be global memory
// or LDS.  Each expert's rank in that order is counted branch-free, width by
// width (one ballot each; groups of 64 experts past E are skipped, a
// wave-uniform test), then one ballot finds the expert of rank `slot`.
// tail > 0 (decode launches on prefill tails): an expert's range is its last
// n mod kPrefillTokTile assignments when fewer than `tail`, else empty.
__device__ __forceinline__ SlotExpert find_slot(const int32_t* offsets, const int (&q)[4], int E, int slot,
                                                int tail = 0)
{
    const int lane = threadIdx.x & 63;
    int lo[4], hi[4], rank[4];
    bool act[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int e = 64 * g + lane;
        const int ec = e < E ? e : 0;
        lo[g] = offsets[ec];
        hi[g] = offsets[ec + 1];
        if (tail > 0) {
            const int r = (hi[g] - lo[g]) % kPrefillTokTile;
            lo[g] = r < tail ? hi[g] - r : hi[g];
        }
        act[g] = e < E && hi[g] > lo[g];
        rank[g] = -1;
    }
    int base = 0;
#pragma unroll
    for (int qq = kQMax; qq >= kQMin; --qq) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            if (64 * g < E) {
                const bool mine = act[g] && q[g] == qq;
                const uint64_t m = __ballot(mine);
                const int r = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                rank[g] = mine ? r : rank[g];
                base += __popcll(m);
            }
        }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const uint64_t hit = __ballot(64 * g < E && rank[g] == slot);
        if (hit) {
            const int h = __ffsll((long long)hit) - 1;
            const int p0 = __builtin_amdgcn_readlane(lo[g], h);
            return SlotExpert{64 * g + h, p0, __builtin_amdgcn_readlane(hi[g], h) - p0};
        }
    }
    return SlotExpert{-1, 0, 0};
}

// Routing mass of one step (PagedWeight pages, Core components 2: online
// routing statistics): expert e's gate weights summed in fp64 in sorted
// (ascending assignment) order, added to mass[e].  Threads take experts;
// offsets, sorted and w may be global memory or LDS.
__device__ __forceinline__ void add_routing_mass(const int32_t* offsets, const int32_t* sorted, const float* w,
                                                 int E, double* mass)
{
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int p0 = offsets[e], p1 = offsets[e + 1];
        if (p1 <= p0) continue;
        double s = 0.0;
        for (int p = p0; p < p1; ++p) s += (double)w[sorted[p]];
        mass[e] += s;
    }
}

__global__ void __launch_bounds__(256) routing_mass_kernel(const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ sorted,
                                                           const float* __restrict__ w, int E, double* mass)
{
    add_routing_mass(offsets, sorted, w, E, mass);
}

__global__ void __launch_bounds__(256) fill_f64_kernel(double* p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.0;
}

// Routing of the whole batch inside a gate_up workgroup (n = T * k <= 64):
// the threads route the tokens (one per lane up to 32 experts, else one per
// wave at a time), wave 0 sorts the assignments.  LDS layout of rt
// (words): idx [64] | w [64] | offsets [257] | sorted [64] | cnt [256] | base [256].
constexpr int kRtIdx = 0, kRtW = 64, kRtOff = 128, kRtSorted = 385, kRtCnt = 449, kRtBase = 705, kRtWords = 961;
static_assert(kRtWords <= kWaves * kSliceWords, "routing scratch lives in the slice region");

__device__ __forceinline__ void route_in_workgroup(const FfnArgs& a, int* rt)
{
    const int wave = threadIdx.x >> 6;
    if (a.E <= kLaneRouteMaxE) {
        const int t = threadIdx.x;  // T <= 64 here
        if (t < a.T) {
            int eo[8];
            float wo[8];
            route_lane_any(a.logits, t, a.E, a.k, eo, wo);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (j < a.k) {
                    rt[kRtIdx + t * a.k + j] = eo[j];
                    ((float*)rt)[kRtW + t * a.k + j] = wo[j];
                }
        }
    } else {
        for (int t = wave; t < a.T; t += kWaves) {
            const RoutePick p = route_pick(a.logits, t, a.E, a.k);
            if (p.j >= 0) {
                rt[kRtIdx + t * a.k + p.j] = p.e;
                ((float*)rt)[kRtW + t * a.k + p.j] = p.w;
            }
        }
    }
    __syncthreads();
    if (wave == 0) sort_small(rt + kRtIdx, a.T * a.k, a.E, rt + kRtOff, rt + kRtSorted, rt + kRtCnt, rt + kRtBase);
    __syncthreads();
}

// y[t][o] of the combine (Problem statement: the layer output is the
// gate-weighted sum of the selected experts' outputs, plus the shared
// expert): routed partial rows of token t summed over the SR K splits, then
// weighted and summed over the picks in pick order, plus the shared row
// summed over its SS K splits.  Every load of the first split (and of up to
// four shared splits) is issued before the first is used (clamped addresses,
// masked sums): one memory round trip instead of one per term.  KM >= k
// picks and SU splits per round trip are compile-time bounds, so a launch with
// few picks or splits issues no clamped duplicate loads (prefill-sized
// batches: a load instruction per term, not the bytes, set the time).
template <int KM, int SU>
__device__ __forceinline__ float combine_value(const FfnArgs& a, int t, int o, int SR, int SS)
{
    const size_t plane = (size_t)a.drows * a.H;
    const float* dr = a.dout + (size_t)t * a.k * a.H + o;                      // token t's routed rows
    const float* ds = SS ? a.dout + ((size_t)a.T * a.k + t) * a.H + o : dr;  // its shared row
    float wj[KM], dj[KM], sv[4];
#pragma unroll
    for (int j = 0; j < KM; ++j) wj[j] = a.topk_w[t * a.k + min(j, a.k - 1)];
#pragma unroll
    for (int j = 0; j < KM; ++j) dj[j] = dr[(size_t)min(j, a.k - 1) * a.H];
#pragma unroll
    for (int u = 0; u < 4; ++u) sv[u] = ds[(size_t)min(u, max(SS - 1, 0)) * plane];
    for (int sp0 = 1; sp0 < SR; sp0 += SU) {
        float v[SU][KM];
#pragma unroll
        for (int u = 0; u < SU; ++u)
#pragma unroll
            for (int j = 0; j < KM; ++j) v[u][j] = dr[(size_t)min(sp0 + u, SR - 1) * plane + (size_t)min(j, a.k - 1) * a.H];
#pragma unroll
        for (int u = 0; u < SU; ++u)
#pragma unroll
            for (int j = 0; j < KM; ++j) dj[j] += sp0 + u < SR ? v[u][j] : 0.0f;
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < KM; ++j) s += j < a.k ? wj[j] * dj[j] : 0.0f;
    if (SS) {
        float sh = 0.0f;
#pragma unroll
        for (int u = 0; u < 4; ++u) sh += u < SS ? sv[u] : 0.0f;
        for (int sp = 4; sp < SS; ++sp) sh += ds[(size_t)sp * plane];
        s += sh;
    }
    return s;
}

// Workgroup order: work units are (row tile, K split) of the shared expert
// first (its work is known to exist and is at the widest width), then of the
// routed slots, slot by slot (slots in decreasing width).  The dispatcher deals
// consecutive workgroups round-robin to the XCDs, so the workgroups that find
// work (slots below the active-expert count) form one contiguous run and every
// XCD gets an equal share of them.  With a.big_wgs > 0 (RG = 4 only) the first
// big_wgs workgroups - one per CU - take whole units and every later unit is
// split into its two 64-row halves (RG = 2 tiles) taken by two workgroups: the
// CUs that get a second workgroup then carry half a unit more, not a whole one.
// FUSED (gate_up only): the launch routes the batch itself (a.logits); the
// workgroup of the first routed unit writes the routing results for the caller
// and for the down and combine launches.
template <int MODE, int RG, bool FUSED = false, bool KEEP = false, int TP = 8>
__global__ void __launch_bounds__(kThreads, 4) ffn_gemv_kernel(FfnArgs a)
{
    __shared__ __align__(16) uint32_t lds[kGemvLdsWords];
    const int wg = blockIdx.x;
    int unit = wg, half = -1;
    if (RG == 4 && a.big_wgs > 0 && wg >= a.big_wgs) {
        const int j = wg - a.big_wgs;
        unit = a.big_wgs + (j >> 1);
        half = j & 1;
    }
    const int shared_units = a.tiles_shared * a.splits_shared;
    bool shared;
    int tile, split, nsplit, p0, ntok, slot_e, tokreg = 0;
    if (unit >= shared_units) {
        shared = false;
        const int rem = unit - shared_units;
        const int per_slot = a.tiles_routed * a.splits_routed;
        const int slot = rem / per_slot;
        const int ts = rem - slot * per_slot;
        tile = ts / a.splits_routed;
        split = ts - tile * a.splits_routed;
        nsplit = a.splits_routed;
        int qw[4];
        load_widths(a.table, MODE, a.E, qw);
        SlotExpert se;
        if constexpr (FUSED) {
            int* rt = (int*)(lds + kLutBytes / 4);
            route_in_workgroup(a, rt);
            const int n = a.T * a.k;
            if (rem == 0 && half <= 0) {
                for (int i = threadIdx.x; i < n; i += kThreads) {
                    a.idx_out[i] = rt[kRtIdx + i];
                    a.w_out[i] = ((const float*)rt)[kRtW + i];
                    a.sorted_out[i] = rt[kRtSorted + i];
                }
                for (int i = threadIdx.x; i <= a.E; i += kThreads) a.offsets_out[i] = rt[kRtOff + i];
                if (a.mass) add_routing_mass(rt + kRtOff, rt + kRtSorted, (const float*)rt + kRtW, a.E, a.mass);
            }
            se = find_slot(rt + kRtOff, qw, a.E, slot);
            tokreg = rt[kRtSorted + min(se.p0 + (int)(threadIdx.x & 63), n - 1)];
            __syncthreads();  // the slice region is reused from here on
        } else {
            se = find_slot(a.offsets, qw, a.E, slot, a.pf_tail);
        }
        if (se.e < 0) return;
        p0 = se.p0;
        ntok = se.ntok;
        slot_e = se.e;
    } else {
        shared = true;
        tile = unit / a.splits_shared;
        split = unit - tile * a.splits_shared;
        nsplit = a.splits_shared;
        p0 = 0;
        ntok = a.T;
        slot_e = a.E;
    }
    const BlockDesc* bd = a.table + (slot_e * 2 + MODE);
    KArgs& ka = kernel_args();
#define PW_GEMV_CASES(RGX, TILE)                                                                                  \
    switch (bd->q) {                                                                                             \
        case 3: mfma_block<MODE, 3, RGX, FUSED, KEEP, TP>(ka, bd, shared, p0, ntok, TILE, split, nsplit, lds, tokreg); break; \
        case 4: mfma_block<MODE, 4, RGX, FUSED, KEEP, TP>(ka, bd, shared, p0, ntok, TILE, split, nsplit, lds, tokreg); break; \
        case 5: mfma_block<MODE, 5, RGX, FUSED, KEEP, TP>(ka, bd, shared, p0, ntok, TILE, split, nsplit, lds, tokreg); break; \
        case 6: mfma_block<MODE, 6, RGX, FUSED, KEEP, TP>(ka, bd, shared, p0, ntok, TILE, split, nsplit, lds, tokreg); break; \
        case 7: mfma_block<MODE, 7, RGX, FUSED, KEEP, TP>(ka, bd, shared, p0, ntok, TILE, split, nsplit, lds, tokreg); break; \
        case 8: mfma_block<MODE, 8, RGX, FUSED, KEEP, TP>(ka, bd, shared, p0, ntok, TILE, split, nsplit, lds, tokreg); break; \
        default: break;                                                                                          \
    }
    if constexpr (RG == 4) {
        if (half >= 0) {
            const int t2 = 2 * tile + half;
            PW_GEMV_CASES(2, t2)
            return;
        }
    }
    PW_GEMV_CASES(RG, tile)
#undef PW_GEMV_CASES
}

// ---------------------------------------------------------------- prefill GEMM
//
// Large token counts per expert (prefill): an expert's contraction is a GEMM
// [tokens x K] x [rows x K]^T on the matrix cores.  One 16-wave workgroup per
// CU owns 128 weight rows (gate_up: 64 gate rows and their 64 up rows; down:
// 128 output rows) x 512 tokens and walks K in 32-column steps (one plane
// word).  The weight and activation tiles of a step live in LDS, double
// buffered: while the waves run the MFMAs of step s, waves 0-7 decode step
// s + 1's weights (each thread: one row, 8 columns, with the same gather and
// LUT look-up as the decode path) and waves 8-15 store the activations of
// step s + 1 (gathered through the expert's assignment list), so decode and
// matrix work overlap and one barrier ends a step.  Global loads run two
// steps ahead.  Both roles put four lanes on one row (a weight row's plane
// word, a token's 64 bytes), so a wave's load touches 2 (planes) or 16
// (activations) cache lines instead of 8 or 64: the vector memory pipeline's
// per-line cost, not the bytes, limited these loads.  Tiles are XOR-swizzled by row so
// the fragment reads and the stores are conflict-free.  Each wave owns 64
// rows x 64 tokens (2 x 2 blocks of v_mfma_f32_32x32x16_f16); a weight is
// decoded once per 512 tokens.  gate_up writes h = silu(g) * u rounded to fp16 (the MFMA operand of
// the down GEMM); down writes the fp32 expert outputs that the combine
// weights and sums.

constexpr int kPfRows = 128;   // weight rows per tile
constexpr int kPfTok = kPrefillTokTile;  // tokens per tile
// 16 waves per prefill workgroup (four per SIMD; 8 is the two-per-SIMD form
// in which every thread both decodes and gathers: 5% slower on the
// Mixtral-shaped prefill layer)
#ifndef PW_PF_WAVES
#define PW_PF_WAVES 16
#endif
constexpr int kPfWaves = PW_PF_WAVES;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfStepCols = 32;  // columns per K step (one plane word)
// LDS words: LUT (64 KB) | weight tiles 2 x [128 rows][4 units] | activation tiles 2 x [512 tokens][4 units]
constexpr int kPfW = kLutBytes / 4;
constexpr int kPfWWords = kPfRows * kPfStepCols / 2;
constexpr int kPfX = kPfW + 2 * kPfWWords;
constexpr int kPfXWords = kPfTok * kPfStepCols / 2;
constexpr int kPfLdsWords = kPfX + 2 * kPfXWords;
static_assert(kPfLdsWords * 4 == 144 * 1024, "prefill LDS: 144 KB");
static_assert(64 * kPfTok <= kPfLdsWords, "epilogue exchanges (64 rows x 512 tokens fp32) fit in LDS");

// Swizzled 16-byte unit u (columns 8u..8u+7 of the step) of tile row r, by
// what gfx950's LDS was measured to do (timed access patterns and the
// SQ_LDS_BANK_CONFLICT counter): a 16-byte read serves 16 lanes per cycle
// over 64 banks, the lanes of a cycle being 0-3, 8-11, 20-23, 28-31 (+32)
// or 0-3, 12-15, 20-23, 24-27 (+32) -- both fit every pattern timed -- and a
// 16-byte write serves 8 consecutive lanes per cycle over 32 banks.  With
// the unit XORed by (r2, r1 ^ r3), the fragment reads (lane l: row
// R0 + l % 32, unit u0 + l / 32) are conflict-free under either read
// grouping, and so are the decoders' tile writes (the same shape) and the
// activation writes (four lanes per token row).  The earlier XOR by
// (r1 ^ r3, r2 ^ r4) conflicted 2-way on the fragment reads.
__device__ __forceinline__ int pf_unit(int r, int u)
{
    return r * 4 + (u ^ (((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1)));
}

// A prefill decoder thread: tile row dr = 16 * (wave % 8) + lane / 4 of a
// 128-row tile (gate_up: rows 0..63 are gate rows i of the tile's 64 h-rows,
// rows 64..127 the matching up rows; down: 128 consecutive rows) and 8-column
// unit dP = lane % 4 of each 32-column step.  Four lanes share a row, so a
// wave's load of a plane word spans 256 contiguous bytes (two cache lines).
// The four lanes of a row read one LUT slot (one bank) at different entries,
// a 4-way conflict on the look-ups; one row per half-wave lane (32 rows x 2
// units per wave) removes it but doubles the cache lines of each plane load,
// and was 10-17% slower.
// LUT slot / half of the row as in the slot layout (gate_up: slot = h-row, up
// rows in the high half; down: slot 32 m + r holds tile rows 64 m + r and
// 64 m + 32 + r); two-set pair tables seed the set bit above the pair code.
struct PfLane {
    int dr, dP, lrow;
    bool valid;
    uint32_t lane_off, acc0;
};

template <int MODE, int Q>
__device__ __forceinline__ PfLane pf_lane(int mtile, int wave, int lane, int R)
{
    PfLane L;
    L.dr = 16 * (wave & 7) + (lane >> 2);
    L.dP = lane & 3;
    int row;
    if (MODE == 0) {
        const int Iblk = R >> 1;
        const int i = mtile * 64 + (L.dr & 63);
        L.valid = i < Iblk;
        row = L.dr < 64 ? i : Iblk + i;
    } else {
        row = mtile * kPfRows + L.dr;
        L.valid = row < R;
    }
    L.lrow = L.valid ? row : 0;
    const int half = MODE == 0 ? L.dr >> 6 : (L.dr >> 5) & 1;
    const int lslot = MODE == 0 ? L.dr & 63 : 32 * (L.dr >> 6) + (L.dr & 31);
    L.lane_off = lut_lane_off<Q, 4>(lslot, half);
    L.acc0 = LutLoad<Q, 4>::PAIR && half ? 0x01010101u << (2 * Q) : 0u;
    return L;
}

// Word index (uint32, within a plane) of step s's word of row `lrow`.
__device__ __forceinline__ size_t pf_word_at(int s, int R, int lrow)
{
    return ((size_t)(s >> 2) * R + lrow) * 4 + (s & 3);
}

// Weights of the lane's unit dP of one plane word set W[p] (an MFMA A
// fragment: element e = column 8 dP + e of the word); *codes receives the
// gathered codes when non-null.
template <int Q, bool PAIR>
__device__ __forceinline__ half8_t pf_decode(const uint32_t (&W)[Q], const PfLane& L, const char* lutb,
                                             StepCodes* codes = nullptr)
{
    Rot<Q, PAIR> rt;
    rotate_planes_lane<Q, PAIR>(W, L.dP, rt);
    const StepCodes c = step_codes_lane<Q, PAIR>(rt, L.acc0);
    StepRaw raw;
    step_lookup<PAIR>(c, L.lane_off, lutb, raw);
    if (codes) *codes = c;
    return step_pack<PAIR>(raw);
}

template <int MODE, int Q, int W>
__device__ __forceinline__ void prefill_block(const KArgs& a, const BlockDesc* __restrict__ bd, bool shared, int p0,
                                              int ntok, int mtile, int ntile, uint32_t* lds, int split = 0,
                                              int nsplit = 1)
{
    constexpr bool PAIR = LutLoad<Q, 4>::PAIR;
    constexpr int NTH = 64 * W;
    // W = 8: every thread decodes one unit and gathers one token row per
    // step.  W = 16: waves 0-7 decode, waves 8-15 gather; every wave does
    // matrix work, so each SIMD runs four waves.
    constexpr bool SPLIT = W == 16;
    constexpr int TB = W == 8 ? 4 : 2;  // 32-token blocks per wave
    constexpr int TS = 32 * TB;         // tokens per wave
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool decoder = !SPLIT || wave < 8;
    const int R = bd->R;
    const int kwords = bd->kwords;
    // K split `split` of nsplit (down): steps k0 .. k0 + nsteps - 1, partial
    // outputs to plane `split` of dout (the combine sums the planes in order)
    const int cps = (kwords + nsplit - 1) / nsplit;
    const int k0 = min(split * cps, kwords);
    const int nsteps = min(kwords - k0, cps);
    const int Iblk = R >> 1;
    const int TK = a.T * a.k;
    // decoder: a wave decodes 16 rows of the tile, four lanes per row (PfLane)
    const PfLane dl = pf_lane<MODE, Q>(mtile, wave, lane, R);
    // activation loader: thread g loads 16-byte unit g % 4 of tile token rows
    // g / 4 + 128 j (j = 0..3), so four neighbouring lanes read one token's 64
    // bytes of a step and a wave's load touches 16 rows instead of 64.  Byte
    // offsets from the x / h base are 32-bit (the launcher checks the bound).
    const int g = tid & 511, gu = g & 3;
    const int n0 = ntile * kPfTok;
    const uintptr_t xbase = MODE == 0 ? (uintptr_t)a.x : (uintptr_t)a.h;
    uint32_t xoff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = 128 * j + (g >> 2);
        const int te = n0 + t < ntok ? n0 + t : n0;
        uint32_t row, stride;
        if (MODE == 0) {
            row = shared ? te : a.sorted[p0 + te] / a.k;
            stride = a.H;
        } else {
            row = shared ? TK + te : p0 + te;
            stride = a.hstride;
        }
        xoff[j] = (row * stride + 8u * gu) * 2u;
    }

    u32x4* wt = (u32x4*)(lds + kPfW);  // [buffer][128 rows x 4 units]
    u32x4* xt = (u32x4*)(lds + kPfX);  // [buffer][512 tokens x 4 units]
    const char* lutb = (const char*)lds;
    const __attribute__((address_space(4))) BlockDesc* cbd =
        (const __attribute__((address_space(4))) BlockDesc*)(uintptr_t)bd;
    const int rb = wave & 1, tb = wave >> 1;  // this wave: 64 rows x TS tokens
    f32x16 C[2][TB];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < TB; ++j) C[i][j] = f32x16{};
    // a wave whose token range holds no token of the tile (the ragged last
    // tile of an expert may hold a few dozen) skips its matrix work (its
    // outputs are never stored); the test is wave-uniform
    const bool nlive = __builtin_amdgcn_readfirstlane(n0 + TS * tb < ntok ? 1 : 0) != 0;

    // The K loop of one role (DW: decode weights, DX: gather activations),
    // so that a thread's registers hold only its own role's loads.  Loads of
    // step s (columns 32 s .. 32 s + 31); two steps are in flight.
    auto run = [&](auto dw_tag, auto dx_tag) {
        constexpr bool DW = decltype(dw_tag)::value, DX = decltype(dx_tag)::value;
        u32x4 xr[2][DX ? 4 : 1];
        uint32_t pw[2][DW ? Q : 1];
        auto issue = [&](int st, int slot) {
            const int s = k0 + min(st, nsteps - 1);
            if constexpr (DX) {
#pragma unroll
                for (int j = 0; j < 4; ++j) xr[slot][j] = *(gcu32x4p)(xbase + (xoff[j] + (uint32_t)s * (2 * kPfStepCols)));
            }
            if constexpr (DW) {
                const size_t at = pf_word_at(s, R, dl.lrow);
                // ordinary (temporal) loads: every token tile of an expert
                // re-reads its planes, and with the plain tile order the next
                // token tile's reads hit the MALL (nontemporal loads: +7%)
#pragma unroll
                for (int p = 0; p < Q; ++p)
                    pw[slot][p] = *((__attribute__((address_space(1))) const uint32_t*)(uintptr_t)cbd->planes[p] + at);
            }
        };
        // step s (loaded in `slot`) -> LDS buffer s & 1
        auto stage = [&](int s, int slot) {
            const int buf = s & 1;
            if constexpr (DW) {
                const half8 A = pf_decode<Q, PAIR>(pw[slot], dl, lutb);
                wt[buf * (kPfWWords / 4) + pf_unit(dl.dr, dl.dP)] = __builtin_bit_cast(u32x4, A);
            }
            if constexpr (DX) {
                // steps past K (padding to an even count) multiply by zero activations
                const bool live = s < nsteps;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    xt[buf * (kPfXWords / 4) + pf_unit(128 * j + (g >> 2), gu)] = live ? xr[slot][j] : u32x4{0, 0, 0, 0};
            }
        };
        {
            LutLoad<Q, 4, NTH> ls;
            ls.issue(bd->lut, bd->slots, mtile * LutLoad<Q, 4, NTH>::NSLOT, lane, wave);
            issue(0, 0);
            issue(1, 1);
            ls.commit(lds, lds + kPfW, lane, wave);  // pair staging in the (idle) weight tiles
            __syncthreads();
        }
        stage(0, 0);
        issue(2, 0);
        __syncthreads();
        // K steps in pairs so the register slots of the loads stay static;
        // the body is branch-free (a branch would make the compiler wait for
        // every load in flight at its join).  After the matrix work of step
        // st: step st + 1 into the other buffer, then the loads of st + 3
        // into the registers just consumed (kept in this order: a load
        // hoisted above the stores would force register copies and a wait
        // for every load in flight).
        for (int s = 0; s < nsteps; s += 2) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int st = s + h;
                const int buf = st & 1;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int u = 2 * kk + (lane >> 5);
                    if (nlive > 0) {
                        half8 Af[2], Bf[TB];
#pragma unroll
                        for (int i = 0; i < 2; ++i)
                            Af[i] = __builtin_bit_cast(half8, wt[buf * (kPfWWords / 4) + pf_unit(64 * rb + 32 * i + (lane & 31), u)]);
#pragma unroll
                        for (int j = 0; j < TB; ++j)
                            Bf[j] = __builtin_bit_cast(half8, xt[buf * (kPfXWords / 4) + pf_unit(TS * tb + 32 * j + (lane & 31), u)]);
#pragma unroll
                        for (int i = 0; i < 2; ++i)
#pragma unroll
                            for (int j = 0; j < TB; ++j)
                                C[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Af[i], Bf[j], C[i][j], 0, 0, 0);
                    }
                }
                stage(st + 1, 1 - h);
                __builtin_amdgcn_sched_barrier(0);
                issue(st + 3, 1 - h);
                __syncthreads();
            }
        }
    };
    // both roles pass the same barriers
    if constexpr (SPLIT) {
        if (decoder) run(std::true_type{}, std::false_type{});
        else run(std::false_type{}, std::true_type{});
    } else {
        run(std::true_type{}, std::true_type{});
    }

    // epilogue; C[i][j][e]: tile row 64 rb + 32 i + 8 (e / 4) + 4 (lane / 32) + e % 4,
    // token n0 + TS tb + 32 j + lane % 32
    if (MODE == 0) {
        float* up = (float*)lds;  // [64 rows][512 tokens]
        if (rb == 1) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < TB; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int r = 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                        up[r * kPfTok + TS * tb + 32 * j + (lane & 31)] = C[i][j][e];
                    }
        }
        __syncthreads();
        // h = silu(g) * u of every entry, in place of g
        if (rb == 0) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < TB; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int r = 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                        const float g = C[i][j][e], u = up[r * kPfTok + TS * tb + 32 * j + (lane & 31)];
                        C[i][j][e] = g / (1.0f + __expf(-g)) * u;
                    }
        }
        __syncthreads();  // `up` is consumed: its LDS holds the fp16 h tile next
        // h tile [512 tokens][32 words], word w = rows 2w (low half) and 2w + 1;
        // the word index is XORed with (t & 7) << 2 so the pair stores of a
        // half-wave (32 tokens) spread over 8 banks and each 8-row group stays
        // 16 contiguous bytes
        uint32_t* hw = lds;
        if (rb == 0) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < TB; ++j)
#pragma unroll
                    for (int e = 0; e < 16; e += 2) {
                        const int w = (32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) >> 1;
                        const int t = TS * tb + 32 * j + (lane & 31);
                        const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)C[i][j][e]);
                        const uint32_t hi16 = __builtin_bit_cast(uint16_t, (_Float16)C[i][j][e + 1]);
                        hw[t * 32 + (w ^ ((t & 7) << 2))] = lo | (hi16 << 16);
                    }
        }
        __syncthreads();
        // stores of whole rows: eight lanes write a token's 64 h entries (128
        // contiguous bytes); I and I_shared are multiples of 32, so an 8-row
        // group is wholly inside or outside the block
#pragma unroll
        for (int k = tid; k < kPfTok * 8; k += kPfThreads) {
            const int t = k >> 3, g8 = k & 7;
            const int hi = mtile * 64 + 8 * g8;
            if (n0 + t < ntok && hi < Iblk) {
                const u32x4 v = *(const u32x4*)&hw[t * 32 + ((4 * g8) ^ ((t & 7) << 2))];
                const int hrow = shared ? TK + n0 + t : p0 + n0 + t;
                *(u32x4*)(a.h + (size_t)hrow * a.hstride + hi) = v;
            }
        }
    } else {
        // two halves of 64 rows: the half's waves stage it in LDS as [512 tokens]
        // [64 rows] fp32 (row index XORed with (t & 15) << 2, which keeps 4-row
        // groups contiguous), then sixteen lanes write each token's 256
        // contiguous bytes of its expert-output row
        float* sto = (float*)lds;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            __syncthreads();  // LDS free: the K loop's (hh 0) or the first half's (hh 1) reads are done
            if (rb == hh) {
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < TB; ++j)
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int r = 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                            const int t = TS * tb + 32 * j + (lane & 31);
                            sto[t * 64 + (r ^ ((t & 15) << 2))] = C[i][j][e];
                        }
            }
            __syncthreads();
#pragma unroll
            for (int k = tid; k < kPfTok * 16; k += kPfThreads) {
                const int t = k >> 4, g4 = k & 15;
                const int row = mtile * kPfRows + 64 * hh + 4 * g4;
                if (n0 + t < ntok && row < R) {
                    const int orow = shared ? TK + n0 + t : a.sorted[p0 + n0 + t];
                    const u32x4 v = *(const u32x4*)&sto[t * 64 + ((4 * g4) ^ ((t & 15) << 2))];
                    *(u32x4*)(a.dout + ((size_t)split * a.drows + orow) * a.H + row) = v;
                }
            }
        }
    }
}

// Workgroups: the shared block's (token tile, row tile) pairs first, then the
// routed ones.  Routed token tiles are numbered over the experts in index
// order (expert e has ceil(ntok_e / 512) of them); workgroups past the last
// tile return at once.  Row tiles are fastest: the chip sweeps the row tiles
// of one token tile together (its activation tile stays in the L2s and the
// MALL), and the next token tile of the same expert re-reads the expert's
// planes from the MALL.  Giving each XCD a contiguous run of this order
// instead was 14% slower.
template <int MODE>
__global__ void __launch_bounds__(kPfThreads, kPfWaves / 4) ffn_prefill_kernel(FfnArgs a)
{
    __shared__ __align__(16) uint32_t lds[kPfLdsWords];
    KArgs& ka = kernel_args();
    const int wg = blockIdx.x;
    // K splits (down): each (token tile, row tile) pair takes nsplit
    // workgroups, row tiles fastest, then splits
    const int nsplit = MODE == 1 ? a.splits_routed : 1;
    const int shared_wgs = a.tiles_shared * a.tok_tiles_shared * nsplit;
    bool shared;
    int mtile, ntile, p0, ntok, e, split;
    if (wg < shared_wgs) {
        shared = true;
        const int per = a.tiles_shared * nsplit;
        ntile = wg / per;
        const int rem = wg - ntile * per;
        split = rem / a.tiles_shared;
        mtile = rem - split * a.tiles_shared;
        p0 = 0;
        ntok = a.T;
        e = a.E;
    } else {
        shared = false;
        const int r = wg - shared_wgs;
        const int per = a.tiles_routed * nsplit;
        const int gn = r / per;
        const int rem = r - gn * per;
        split = rem / a.tiles_routed;
        mtile = rem - split * a.tiles_routed;
        // expert of routed token tile gn: inclusive scan of the tile counts
        const int lane = threadIdx.x & 63;
        int base = 0;
        e = -1;
        ntile = 0;
        p0 = 0;
        ntok = 0;
        for (int g = 0; g < (a.E + 63) / 64; ++g) {
            const int ee = 64 * g + lane;
            const int lo = ee < a.E ? a.offsets[ee] : 0, hi = ee < a.E ? a.offsets[ee + 1] : 0;
            // token tiles of the expert (a short tail is left to the decode launches)
            const int n = hi - lo;
            const int cnt = a.pf_tail > 0 ? n / kPfTok + (n % kPfTok >= a.pf_tail ? 1 : 0) : (n + kPfTok - 1) / kPfTok;
            const int incl = wave_inclusive_sum(cnt);
            const int excl = base + incl - cnt;
            const uint64_t hit = __ballot(cnt > 0 && gn >= excl && gn < excl + cnt);
            if (hit) {
                const int h = __ffsll((long long)hit) - 1;
                e = 64 * g + h;
                ntile = gn - __shfl(excl, h);
                p0 = __shfl(lo, h);
                ntok = __shfl(hi, h) - p0;
                break;
            }
            base += __shfl(incl, 63);
        }
        e = __builtin_amdgcn_readfirstlane(e);
        if (e < 0) return;
        ntile = __builtin_amdgcn_readfirstlane(ntile);
        p0 = __builtin_amdgcn_readfirstlane(p0);
        ntok = __builtin_amdgcn_readfirstlane(ntok);
    }
    const BlockDesc* bd = a.table + (e * 2 + MODE);
    switch (bd->q) {
        case 3: prefill_block<MODE, 3, kPfWaves>(ka, bd, shared, p0, ntok, mtile, ntile, lds, split, nsplit); break;
        case 4: prefill_block<MODE, 4, kPfWaves>(ka, bd, shared, p0, ntok, mtile, ntile, lds, split, nsplit); break;
        case 5: prefill_block<MODE, 5, kPfWaves>(ka, bd, shared, p0, ntok, mtile, ntile, lds, split, nsplit); break;
        case 6: prefill_block<MODE, 6, kPfWaves>(ka, bd, shared, p0, ntok, mtile, ntile, lds, split, nsplit); break;
        case 7: prefill_block<MODE, 7, kPfWaves>(ka, bd, shared, p0, ntok, mtile, ntile, lds, split, nsplit); break;
        case 8: prefill_block<MODE, 8, kPfWaves>(ka, bd, shared, p0, ntok, mtile, ntile, lds, split, nsplit); break;
        default: break;
    }
}

// y[t][o] = sum_j w[t][j] * (sum over splits of d_(t,j)[o]) (+ shared d), rounded once to fp16.
template <int KM, int SU>
__global__ void __launch_bounds__(256) combine_kernel(FfnArgs a)
{
    // grid: (token, 256-column group of H)
    const int t = blockIdx.x, o = blockIdx.y * 256 + threadIdx.x;
    if (o >= a.H) return;
    const float v = combine_value<KM, SU>(a, t, o, a.splits_routed, a.tiles_shared ? a.splits_shared : 0);
    a.y[(size_t)t * a.H + o] = __builtin_bit_cast(uint16_t, (_Float16)v);
}

// ---------------------------------------------------------------- debug export
//
// The decode of one block exactly as the FFN kernels run it, with the codes
// and weights written out instead of multiplied: the same LUT staging
// (LutLoad), lane geometry (tile_lane / pf_lane), plane loads
// (load_pair_words / pf_word_at) and code gather and look-up (WordDecoder,
// step_lookup, step_pack / pf_decode).  Outputs are row-major [R][K] (codes
// uint8, weights fp16 bits); either may be null.

// The 8 codes and weights of one MFMA step of row `row` (columns col..col+7;
// columns past K -- the zero words of a partial last chunk -- are skipped).
template <int Q, bool PAIR>
__device__ __forceinline__ void debug_store_step(const StepCodes& c, const half8_t& A, int row, int col, int K,
                                                 uint8_t* codes_out, uint16_t* w_out)
{
    if (col >= K) return;
    const size_t base = (size_t)row * K + col;
    const u32x4 wv = __builtin_bit_cast(u32x4, A);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t ca, cb;
        if constexpr (PAIR) {
            const uint32_t pr = (c.c0 >> (8 * i)) & 0xffu;
            ca = pr & ((1u << Q) - 1u);
            cb = (pr >> Q) & ((1u << Q) - 1u);
        } else {
            ca = (c.c0 >> (8 * i)) & 0xffu;
            cb = (c.c1 >> (8 * i)) & 0xffu;
        }
        if (codes_out) {
            codes_out[base + 2 * i] = (uint8_t)ca;
            codes_out[base + 2 * i + 1] = (uint8_t)cb;
        }
        if (w_out) {
            w_out[base + 2 * i] = (uint16_t)(wv[i] & 0xffffu);
            w_out[base + 2 * i + 1] = (uint16_t)(wv[i] >> 16);
        }
    }
}

// One decode-contraction tile (8 waves, RG row groups, as mfma_block; WIDE:
// the tables of 16- and 32-token passes).
template <int MODE, int Q, int RG, bool WIDE = false>
__device__ void debug_gemv_tile(const BlockDesc* __restrict__ bd, int tile, uint8_t* codes_out, uint16_t* w_out,
                                uint32_t* lds)
{
    constexpr int KW = kWaves / RG;
    constexpr bool PAIR = LutLoad<Q, RG, kThreads, WIDE>::PAIR;
    const int tid = threadIdx.x, lane = tid & 63, rho = lane & 31, kh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave / KW, kw = wave % KW;
    const int R = bd->R, K = bd->kwords * 32, nchunks = bd->nchunks;
    const TileLane tl = tile_lane<MODE, Q, RG, WIDE>(tile, grp, rho, R);
    {
        LutLoad<Q, RG, kThreads, WIDE> ls;
        ls.issue(bd->lut, bd->slots, tile * LutLoad<Q, RG, kThreads, WIDE>::NSLOT, lane, wave);
        ls.commit(lds, lds + kLutBytes / 4, lane, wave);
        __syncthreads();
    }
    WordDecoder<Q, RG, WIDE> dec;
    dec.masks = make_masks();
    dec.zero = (uint32_t)__builtin_amdgcn_readfirstlane(R >> 30);  // R < 2^30
    dec.set1 = tl.set1;
    const char* lutb = (const char*)lds;
    for (int c = kw; c < nchunks; c += KW) {
        u32x2 pg[Q];
        load_pair_words<Q>(pg, bd, c, R, tl.lrow, kh);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            uint32_t W[Q];
#pragma unroll
            for (int p = 0; p < Q; ++p) W[p] = pg[p][u];
            dec.prepare(W);
#pragma unroll
            for (int P = 0; P < 4; ++P) {
                const StepCodes sc = dec.codes(P);
                StepRaw raw;
                step_lookup<PAIR>(sc, tl.lane_off, lutb, raw);
                const half8_t A = step_pack<PAIR>(raw);
                if (tl.valid)
                    debug_store_step<Q, PAIR>(sc, A, tl.row, c * kChunkCols + 32 * (2 * kh + u) + 8 * P, K, codes_out,
                                              w_out);
            }
        }
    }
}

// One prefill tile's decoder waves (16-wave workgroup, as prefill_block).
template <int MODE, int Q>
__device__ void debug_prefill_tile(const BlockDesc* __restrict__ bd, int mtile, uint8_t* codes_out, uint16_t* w_out,
                                   uint32_t* lds)
{
    constexpr bool PAIR = LutLoad<Q, 4>::PAIR;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int R = bd->R, K = bd->kwords * 32;
    {
        LutLoad<Q, 4, kPfThreads> ls;
        ls.issue(bd->lut, bd->slots, mtile * LutLoad<Q, 4, kPfThreads>::NSLOT, lane, wave);
        ls.commit(lds, lds + kPfW, lane, wave);
        __syncthreads();
    }
    if (wave >= 8) return;  // the gatherer waves
    const PfLane dl = pf_lane<MODE, Q>(mtile, wave, lane, R);
    const __attribute__((address_space(4))) BlockDesc* cbd =
        (const __attribute__((address_space(4))) BlockDesc*)(uintptr_t)bd;
    const char* lutb = (const char*)lds;
    for (int s = 0; s < bd->kwords; ++s) {
        const size_t at = pf_word_at(s, R, dl.lrow);
        uint32_t W[Q];
#pragma unroll
        for (int p = 0; p < Q; ++p) W[p] = *((__attribute__((address_space(1))) const uint32_t*)(uintptr_t)cbd->planes[p] + at);
        StepCodes sc;
        const half8_t A = pf_decode<Q, PAIR>(W, dl, lutb, &sc);
        if (dl.valid) debug_store_step<Q, PAIR>(sc, A, dl.lrow, 32 * s + 8 * dl.dP, K, codes_out, w_out);
    }
}

constexpr int kDebugPfLdsWords = kPfX;  // LUT + the weight tiles (pair-table staging)

// PATH 0 / 1: decode contraction with RG = 4 / RG = 2 tiles; PATH 2: prefill
// decoder; PATH 3: RG = 2 tiles of 16- and 32-token passes.  One workgroup per tile
// of that path.
template <int PATH>
__global__ void __launch_bounds__(PATH == 2 ? kPfThreads : kThreads)
    debug_decode_kernel(const BlockDesc* __restrict__ bd, int module, uint8_t* codes_out, uint16_t* w_out)
{
    __shared__ __align__(16) uint32_t lds[PATH == 2 ? kDebugPfLdsWords : kGemvLdsWords];
    const int tile = blockIdx.x;
#define PW_DEBUG_CASE(M, QQ)                                                                        \
    case 2 * (QQ) + (M):                                                                            \
        if constexpr (PATH == 2) debug_prefill_tile<M, QQ>(bd, tile, codes_out, w_out, lds);        \
        else debug_gemv_tile<M, QQ, PATH == 0 ? 4 : 2, PATH == 3>(bd, tile, codes_out, w_out, lds); \
        break;
    switch (2 * bd->q + module) {
        PW_DEBUG_CASE(0, 3) PW_DEBUG_CASE(1, 3) PW_DEBUG_CASE(0, 4) PW_DEBUG_CASE(1, 4)
        PW_DEBUG_CASE(0, 5) PW_DEBUG_CASE(1, 5) PW_DEBUG_CASE(0, 6) PW_DEBUG_CASE(1, 6)
        PW_DEBUG_CASE(0, 7) PW_DEBUG_CASE(1, 7) PW_DEBUG_CASE(0, 8) PW_DEBUG_CASE(1, 8)
        default: break;
    }
#undef PW_DEBUG_CASE
}

// ---------------------------------------------------------------- width changes
//
// Page movement of a width change (Core components 3: pages move
// asynchronously, widths are committed at safe boundaries) in a few launches,
// so a change of hundreds of blocks costs the host a few calls instead of one
// copy per plane and per page-table entry.

// The copies of a list (pinned host memory, read through its device-side
// address); every size is a multiple of 16 bytes.  Two uses: the copies of a
// blocking width change straight from the pinned host masters (bound by the
// host link: a few workgroups, one copy each at a time), and the scatter of a
// staging chunk that one DMA brought to the device into the new plane and LUT
// slabs (a short burst: each copy split in `parts` byte ranges, one
// workgroup each).  8 x 16 bytes per thread in flight.
constexpr int kPullWgs = 16;
__global__ void __launch_bounds__(256) pull_copy_kernel(const CopyDesc* __restrict__ list, int n, int parts)
{
    constexpr int U = 8;
    for (int j = blockIdx.x; j < n * parts; j += gridDim.x) {
        const int item = j / parts, part = j - item * parts;
        const CopyDesc d = list[item];
        const u32x4* src = (const u32x4*)d.src;
        u32x4* dst = (u32x4*)d.dst;
        const uint64_t n16 = d.bytes / 16;
        const uint64_t lo = n16 * part / parts, hi = n16 * (part + 1) / parts;
        for (uint64_t i = lo + threadIdx.x; i < hi; i += U * 256) {
            u32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint64_t at = i + (uint64_t)u * 256;
                v[u] = at < hi ? src[at] : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint64_t at = i + (uint64_t)u * 256;
                if (at < hi) dst[at] = v[u];
            }
        }
    }
}

// Commit of new page-table entries: descs[i] (pinned host memory) ->
// table[ids[i]], eight threads per 128-byte entry.
__global__ void __launch_bounds__(256) scatter_desc_kernel(BlockDesc* __restrict__ table, const int32_t* __restrict__ ids,
                                                           const BlockDesc* __restrict__ descs, int n)
{
    const int i = blockIdx.x * 32 + (threadIdx.x >> 3), part = threadIdx.x & 7;
    if (i < n) ((u32x4*)(table + ids[i]))[part] = ((const u32x4*)(descs + i))[part];
}

// ---------------------------------------------------------------- static scratch
//
// Workspace of the allocation-free layer entry point: file-scope device
// memory, one copy per GPU, held until the process ends.  Host code never
// passes the array's name to a kernel (in host code it is a stand-in, not a
// device address): static_scratch() looks up each device's address once,
// with that device current, and every later use goes through it.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

hipError_t static_scratch(int device, void** out)
{
    static std::mutex mu;
    static void* ptrs[kMaxDevices] = {};
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[device]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        ptrs[device] = p;
    }
    *out = ptrs[device];
    return hipSuccess;
}

// ---------------------------------------------------------------- launchers

thread_local LaunchEvents* launch_events = nullptr;

template <typename Kern, typename... Args>
static void launch(Kern kernel, dim3 grid, dim3 block, hipStream_t s, Args... args)
{
    LaunchEvents* ev = launch_events;
    if (ev && !ev->used) {
        ev->used = true;
        hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev->start, ev->stop, 0, args...);
    } else {
        hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
    }
}


hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w, hipStream_t s)
{
    if (E <= kLaneRouteMaxE)
        launch(route_topk_lane_kernel, dim3((T + 255) / 256), dim3(256), s, logits, T, E, k, idx, w);
    else
        launch(route_topk_kernel, dim3((T + 3) / 4), dim3(256), s, logits, T, E, k, idx, w);
    return hipGetLastError();
}

hipError_t launch_route_permute(const float* logits, int T, int E, int k, int32_t* idx, float* w, int32_t* offsets,
                                int32_t* sorted, hipStream_t s)
{
    launch(route_permute_kernel, dim3(1), dim3(1024), s, logits, T, E, k, idx, w, offsets, sorted);
    return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets, int32_t* sorted,
                          hipStream_t s)
{
    launch(permute_kernel, dim3(1), dim3(1024), s, idx, T * k, E, offsets, sorted);
    return hipGetLastError();
}

// workgroups of a decode launch: every unit, plus one more per unit past the
// first big_wgs when those units are split in halves
static int gemv_grid(const FfnArgs& a)
{
    const int units = a.n_slots * a.tiles_routed * a.splits_routed + a.tiles_shared * a.splits_shared;
    if (a.rg == 4 && a.big_wgs > 0 && units > a.big_wgs) return a.big_wgs + 2 * (units - a.big_wgs);
    return units;
}

hipError_t launch_gate_up(const FfnArgs& a, hipStream_t s)
{
    const int grid = gemv_grid(a);
    if (grid == 0) return hipSuccess;
    if (a.tok_pass == 16 || a.tok_pass == 32) {
        if (a.logits || (a.tok_pass == 16 && a.rg != 2)) return hipErrorInvalidValue;
        if (a.tok_pass == 32) {
            if (a.rg == 4) {
                if (a.keep_planes)
                    launch((ffn_gemv_kernel<0, 4, false, true, 32>), dim3(grid), dim3(kThreads), s, a);
                else
                    launch((ffn_gemv_kernel<0, 4, false, false, 32>), dim3(grid), dim3(kThreads), s, a);
            } else if (a.keep_planes)
                launch((ffn_gemv_kernel<0, 2, false, true, 32>), dim3(grid), dim3(kThreads), s, a);
            else
                launch((ffn_gemv_kernel<0, 2, false, false, 32>), dim3(grid), dim3(kThreads), s, a);
        } else if (a.keep_planes)
            launch((ffn_gemv_kernel<0, 2, false, true, 16>), dim3(grid), dim3(kThreads), s, a);
        else
            launch((ffn_gemv_kernel<0, 2, false, false, 16>), dim3(grid), dim3(kThreads), s, a);
    } else if (a.logits) {
        if (a.rg != 4 || a.T * a.k > kLayerRouteMaxAssign || a.E > 256) return hipErrorInvalidValue;
        launch((ffn_gemv_kernel<0, 4, true>), dim3(grid), dim3(kThreads), s, a);
    } else if (a.rg == 4) {
        if (a.keep_planes)
            launch((ffn_gemv_kernel<0, 4, false, true>), dim3(grid), dim3(kThreads), s, a);
        else
            launch((ffn_gemv_kernel<0, 4>), dim3(grid), dim3(kThreads), s, a);
    } else {
        launch((ffn_gemv_kernel<0, 2>), dim3(grid), dim3(kThreads), s, a);
    }
    return hipGetLastError();
}

hipError_t launch_down(const FfnArgs& a, hipStream_t s)
{
    const int grid = gemv_grid(a);
    if (grid == 0) return hipSuccess;
    if (a.tok_pass == 16 || a.tok_pass == 32) {
        if (a.rg != 2) return hipErrorInvalidValue;
        if (a.tok_pass == 32) {
            if (a.keep_planes)
                launch((ffn_gemv_kernel<1, 2, false, true, 32>), dim3(grid), dim3(kThreads), s, a);
            else
                launch((ffn_gemv_kernel<1, 2, false, false, 32>), dim3(grid), dim3(kThreads), s, a);
        } else if (a.keep_planes)
            launch((ffn_gemv_kernel<1, 2, false, true, 16>), dim3(grid), dim3(kThreads), s, a);
        else
            launch((ffn_gemv_kernel<1, 2, false, false, 16>), dim3(grid), dim3(kThreads), s, a);
    } else if (a.rg == 4)
        launch((ffn_gemv_kernel<1, 4>), dim3(grid), dim3(kThreads), s, a);
    else if (a.keep_planes)
        launch((ffn_gemv_kernel<1, 2, false, true>), dim3(grid), dim3(kThreads), s, a);
    else
        launch((ffn_gemv_kernel<1, 2>), dim3(grid), dim3(kThreads), s, a);
    return hipGetLastError();
}

hipError_t launch_prefill(const FfnArgs& a, int module, hipStream_t s)
{
    const int nsplit = module == 1 ? a.splits_routed : 1;
    if (nsplit < 1 || (module == 1 && a.splits_shared != nsplit)) return hipErrorInvalidValue;
    const int grid = (a.tiles_shared * a.tok_tiles_shared + a.tiles_routed * a.tok_tiles_routed) * nsplit;
    if (grid == 0) return hipSuccess;
    if (module == 0)
        launch(ffn_prefill_kernel<0>, dim3(grid), dim3(kPfThreads), s, a);
    else
        launch(ffn_prefill_kernel<1>, dim3(grid), dim3(kPfThreads), s, a);
    return hipGetLastError();
}

hipError_t launch_combine(const FfnArgs& a, hipStream_t s)
{
    if (a.T <= 0 || a.H <= 0) return hipSuccess;
    const dim3 grid((unsigned)a.T, (unsigned)((a.H + 255) / 256));
    // picks bound 2 / 4 / 8; routed splits one (<= 2) or four per round trip
    if (a.k > 8) return hipErrorInvalidValue;
    const bool su1 = a.splits_routed <= 2;
    if (a.k <= 2) {
        if (su1) launch((combine_kernel<2, 1>), grid, dim3(256), s, a);
        else launch((combine_kernel<2, 4>), grid, dim3(256), s, a);
    } else if (a.k <= 4) {
        if (su1) launch((combine_kernel<4, 1>), grid, dim3(256), s, a);
        else launch((combine_kernel<4, 4>), grid, dim3(256), s, a);
    } else if (su1) {
        launch((combine_kernel<8, 1>), grid, dim3(256), s, a);
    } else {
        launch((combine_kernel<8, 4>), grid, dim3(256), s, a);
    }
    return hipGetLastError();
}

hipError_t launch_routing_mass(const int32_t* offsets, const int32_t* sorted, const float* w, int E, double* mass,
                               hipStream_t s)
{
    launch(routing_mass_kernel, dim3(1), dim3(256), s, offsets, sorted, w, E, mass);
    return hipGetLastError();
}

hipError_t launch_fill_f64(double* p, int64_t n, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    launch(fill_f64_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), s, p, n);
    return hipGetLastError();
}

hipError_t launch_pull_copy(const CopyDesc* list, int n, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    launch(pull_copy_kernel, dim3((unsigned)std::min(n, kPullWgs)), dim3(256), s, list, n, 1);
    return hipGetLastError();
}

hipError_t launch_scatter_copy(const CopyDesc* list, int n, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    constexpr int kScatterWgs = 512;
    const int parts = std::max(1, kScatterWgs / n);
    launch(pull_copy_kernel, dim3((unsigned)std::min(n * parts, kScatterWgs)), dim3(256), s, list, n, parts);
    return hipGetLastError();
}

hipError_t launch_scatter_desc(BlockDesc* table, const int32_t* ids, const BlockDesc* descs, int n, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    launch(scatter_desc_kernel, dim3((unsigned)((n + 31) / 32)), dim3(256), s, table, ids, descs, n);
    return hipGetLastError();
}

hipError_t launch_debug_decode(const BlockDesc* entry, int module, int R, int path, uint8_t* codes_out,
                               uint16_t* w_out, hipStream_t s)
{
    const int rows = module == 0 ? R / 2 : R;  // gate_up tiles count h-rows
    if (path == 2) {
        const int per = module == 0 ? kPfRows / 2 : kPfRows;
        launch(debug_decode_kernel<2>, dim3((rows + per - 1) / per), dim3(kPfThreads), s, entry, module, codes_out,
               w_out);
    } else {
        const int rg = path == 0 ? 4 : 2;
        const int per = module == 0 ? 16 * rg : 32 * rg;
        const dim3 grid((rows + per - 1) / per);
        if (path == 0)
            launch(debug_decode_kernel<0>, grid, dim3(kThreads), s, entry, module, codes_out, w_out);
        else if (path == 1)
            launch(debug_decode_kernel<1>, grid, dim3(kThreads), s, entry, module, codes_out, w_out);
        else
            launch(debug_decode_kernel<3>, grid, dim3(kThreads), s, entry, module, codes_out, w_out);
    }
    return hipGetLastError();
}

}  // namespace pw
