// Device-side numerical contract shared by every attention kernel of the
// library.  Output bits of a query row depend only on (q row, K/V rows
// 0..pos, scale): every kernel reaches them through the functions in this
// header, with the same operand layouts, reduction orders and instructions.
//
// The pages (KernelBraid / AReaL-TIK README, "Method" and "Advantages") fix
// only the property: full-sequence prefill, partitioned forward and one-token
// decode agree bit for bit, with tiling, data movement, parallelism and
// dispatch free inside one contract.  This header is that contract for gfx950:
//
//   tile    T = 64 keys, absolute boundaries at multiples of 64 from key 0
//   chunk   C = 1024 keys (16 tiles): the unit of the fold and of split-KV
//   MFMA    v_mfma_f32_32x32x16_bf16 for both products:
//             S^T[key][query] = K[key][:] . Q^T[:][query]     (A = K, B = Q^T)
//             O^T[d][query]  += V^T[d][keys] . P^T[keys][query] (A = V^T, B = P^T)
//           one query per MFMA column; column position never changes bits.
//   per row, per tile, in order (running state mc = reference max * c, l, o):
//     s_j   = MFMA chain over d in k-steps 0..7 (step st covers d 16st..16st+15)
//     s_j   = -inf where key j > pos                  (select)
//     mtc   = (max_j s_j) * c                         with c = fp32(scale * log2 e)
//     grow  = mtc - mc > 64;  mc' = grow ? mtc : mc;  a = grow ? exp2(mc - mc') : 1
//     p_j   = exp2(fma(s_j, c, -mc'));  P_j = bf16_rne(p_j)   (P_j <= 2^64)
//     l     = fma(l, a, sum(P))   sum: per lane half, one chain of 16 bf16
//             dot2 with (1, 1) over the key steps (0,0), (0,1), (1,0), (1,1)
//             in order, 4 per step; then (low half + high half)
//     o     = o * a;  o = MFMA chain over the tile's 4 key steps in order
//     mc    = mc'
//   per chunk, in chunk order (first chunk is copied, the rest folded):
//     Mc' = max(Mc, mc); A = (Mc' == Mc) ? 1 : exp2(Mc - Mc')
//     B   = (Mc' == mc) ? 1 : exp2(mc - Mc'); L = fma(L, A, l B); O = fma(O, A, o B)
//   out = bf16_rne(q), q = O / L by reciprocal and one correction (finalize)
//   lse = (Mc + log2(L)) * fp32(ln 2)   (v_log_f32; natural-log log-sum-exp
//         of the scaled scores, emitted on request from the same (Mc, L))
//
// Compile every kernel of the library in one translation unit with
// -ffp-contract=off so that no multiply-add is fused behind the contract's back.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kb {

constexpr int kHeadDim = 128;
constexpr int kTile = 64;
constexpr int kChunk = 1024;
constexpr int kTilesPerChunk = kChunk / kTile;
constexpr int kGroup = 4;  // query heads per KV head

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Unpadded K/V tile sizes (64 keys x 256 B rows each); the backward kernels
// stage their tiles in this size with layouts of their own.
constexpr int kKBytes = kTile * kHeadDim * 2;
constexpr int kVBytes = kTile * kHeadDim * 2;
constexpr int kTileBytes = kKBytes + kVBytes;
constexpr int kTileLoads = kTileBytes / 1024;  // 32 one-KiB direct loads

__device__ __forceinline__ bf16x8 lds_read16(const char* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ bf16x8 tr_pair(const char* p0, const char* p1) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 all = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, all);
}

// ---------------------------------------------------------------------------
// LDS layouts of one K/V tile (one stage of a ring): K, then V.  Which one a
// kernel uses changes no value it reads, so no bit of any output.  Both are
// filled by one-KiB direct loads (global_load_lds_dwordx4): lane L of load i
// lands at byte 1024 i + 16 L of the stage and fetches the 16-byte chunk of K
// or V that belongs there.  The fragment readers, for every layout:
//   k_frag   A operand of S^T = K Q^T for key block kb, k-step st:
//            lane (key j, half h) holds K[32kb + j][16st + 8h .. +7]
//   vt_frag  A operand of O^T += V^T P^T for key step (kb, u), d block dblk:
//            lane (d = 32 dblk + j, half h) holds, in slot order,
//            V[K0 + 4h + {0..3}][d], V[K0 + 8 + 4h + {0..3}][d], K0 = 32kb + 16u,
//            read with two ds_read_b64_tr_b16.  Within each 16-lane group,
//            lane i of the result takes element (i & 3) of the 8-byte blocks
//            read by lanes 4n + (i >> 2) (n = 0..3), so lane L = 16 g + 4 n + jj
//            reads V[K0 + 4 (g >> 1) + n][32 dblk + 16 (g & 1) + 4 jj .. +3].
// ---------------------------------------------------------------------------

// Padded rows (the prefill): every fragment read is a per-lane base plus a
// constant, so no address arithmetic runs per tile.
//   K  key row r at r * 272 bytes (16 B of padding): the 16 rows read by 16
//      lanes of one A-operand read start 68 words apart, i.e. in 16 distinct
//      groups of 4 banks
//   V  key row r at r * 320 bytes (64 B of padding): a transposing read
//      touches 4 rows x 32 B per 32 lanes, rows 80 words apart, i.e. all 64
//      banks once
// 37 loads per stage (17 for K, 20 for V); padding slots fetch chunk 15 of
// their row, which nothing reads.
struct PaddedTile {
    static constexpr int kKRow = 272;
    static constexpr int kVRow = 320;
    static constexpr int kKStage = kTile * kKRow;  // 17408
    static constexpr int kBytes = kKStage + kTile * kVRow;  // 37888
    static constexpr int kLoads = kBytes / 1024;  // 37
    static constexpr int kKLoads = kKStage / 1024;  // 17

    // source offset, from the tile's first key row, of load i, lane `lane`
    __device__ static __forceinline__ uint32_t src(int i, int lane, int& row, bool& v) {
        v = i >= kKLoads;
        const int p = (v ? i - kKLoads : i) * 64 + lane;  // 16-byte slot in the operand
        const int per = v ? kVRow / 16 : kKRow / 16;       // slots per row (20 or 17)
        row = p / per;
        const int c = min(p - row * per, 15);
        return (uint32_t)(row * 256 + c * 16);
    }
    __device__ static __forceinline__ bf16x8 k_frag(const char* sK, int kb, int st, int lane) {
        const char* base = sK + (lane & 31) * kKRow + (lane >> 5) * 16;
        return lds_read16(base + kb * 32 * kKRow + st * 32);
    }
    __device__ static __forceinline__ bf16x8 vt_frag(const char* sV, int kb, int u, int dblk, int lane) {
        const int g = lane >> 4, n = (lane >> 2) & 3, jj = lane & 3;
        const char* base = sV + (4 * (g >> 1) + n) * kVRow + (16 * (g & 1) + 4 * jj) * 2;
        const char* p0 = base + (32 * kb + 16 * u) * kVRow + 64 * dblk;
        return tr_pair(p0, p0 + 8 * kVRow);
    }
};

// Swizzled 256-byte rows (the decode, which streams HBM and wants the fewest
// loads per tile): 32 loads per stage.
//   K  16-byte chunk c of key row r at chunk position c ^ (r & 15) (the
//      A-operand reads, 16 rows x one chunk per 16 lanes, hit 16 distinct
//      bank groups)
//   V  16-byte chunk c of key row r at chunk position c ^ ((r & 3) << 2)
//      (the transposing reads touch 4 rows x 4 chunks per 32 lanes)
struct SwizzledTile {
    static constexpr int kKStage = kTile * 256;
    static constexpr int kBytes = 2 * kKStage;  // 32768
    static constexpr int kLoads = kBytes / 1024;  // 32
    static constexpr int kKLoads = kKStage / 1024;  // 16

    __device__ static __forceinline__ int k_swz(int row) { return row & 15; }
    __device__ static __forceinline__ int v_swz(int row) { return (row & 3) << 2; }
    __device__ static __forceinline__ uint32_t src(int i, int lane, int& row, bool& v) {
        v = i >= kKLoads;
        row = 4 * (i & 15) + (lane >> 4);
        const int c = (lane & 15) ^ (v ? v_swz(row) : k_swz(row));
        return (uint32_t)(row * 256 + c * 16);
    }
    __device__ static __forceinline__ bf16x8 k_frag(const char* sK, int kb, int st, int lane) {
        const int row = 32 * kb + (lane & 31);
        const int c = 2 * st + (lane >> 5);
        return lds_read16(sK + row * 256 + ((c ^ k_swz(row)) << 4));
    }
    __device__ static __forceinline__ bf16x8 vt_frag(const char* sV, int kb, int u, int dblk, int lane) {
        const int g = lane >> 4, n = (lane >> 2) & 3, jj = lane & 3;
        const int row0 = 32 * kb + 16 * u + 4 * (g >> 1) + n;
        const int d = 32 * dblk + 16 * (g & 1) + 4 * jj;
        const int c = d >> 3, half = (d & 4) << 1;  // byte offset 0 or 8 inside the chunk
        const int row1 = row0 + 8;
        return tr_pair(sV + row0 * 256 + ((c ^ v_swz(row0)) << 4) + half,
                       sV + row1 * 256 + ((c ^ v_swz(row1)) << 4) + half);
    }
};

// Per-wave plan of the direct loads of a stage for a workgroup of NW waves:
// wave w issues loads i = w, w + NW, ... < L::kLoads.  off[k] is lane L's
// source offset for its k-th load; it does not depend on the tile.
template <class L, int NW>
struct StagePlan {
    static constexpr int kN = (L::kLoads + NW - 1) / NW;
    uint32_t off[kN];
};

template <class L, int NW>
__device__ __forceinline__ void stage_plan(StagePlan<L, NW>& p, int lane, int wave) {
#pragma unroll
    for (int k = 0; k < StagePlan<L, NW>::kN; ++k) {
        const int i = wave + k * NW;
        int row;
        bool v;
        p.off[k] = i < L::kLoads ? L::src(i, lane, row, v) : 0u;
    }
}

__device__ __forceinline__ void lds_dma16(const char* sbase, uint32_t voff, const char* dst) {
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    uint32_t saved_m0;
    // M0 is saved and restored around the load; s_nop covers the one wait
    // state required between an M0 write and an LDS-DMA load
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved_m0)
        : "v"(voff), "s"(sbase), "s"(lds_base)
        : "memory");
}

__device__ __forceinline__ void lds_dma16_flat(const void* src, const char* dst) {
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    uint32_t saved_m0;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved_m0)
        : "v"(src), "s"(lds_base)
        : "memory");
}

// Issue this wave's loads of the tile starting at key0 into the stage at
// `stage` (K at stage, V at stage + L::kKStage).  A tile wholly below kv_len
// takes the planned offsets from a scalar tile base; otherwise keys at or
// beyond kv_len read the (valid) row kv_len - 1 instead: those keys are
// masked (K) or weighted by P = 0 (V), so only finite values ever enter the
// products.  The loads are inline assembly so that the compiler does not
// serialise later LDS reads behind them; completion is tracked with wait_vm()
// before the workgroup barrier that publishes the tile.
template <class L, int NW>
__device__ __forceinline__ void stage_tile(const StagePlan<L, NW>& p, const uint16_t* kbase, const uint16_t* vbase,
                                           int64_t key0, int64_t kv_len, char* stage, int lane, int wave) {
    const char* kt = reinterpret_cast<const char*>(kbase + key0 * kHeadDim);
    const char* vt = reinterpret_cast<const char*>(vbase + key0 * kHeadDim);
    if (key0 + kTile <= kv_len) {
#pragma unroll
        for (int k = 0; k < StagePlan<L, NW>::kN; ++k) {
            const int i = wave + k * NW;
            if (k == StagePlan<L, NW>::kN - 1 && i >= L::kLoads) break;
            lds_dma16(i >= L::kKLoads ? vt : kt, p.off[k], stage + 1024 * i);
        }
    } else {
        for (int i = wave; i < L::kLoads; i += NW) {
            int row;
            bool v;
            const uint32_t off = L::src(i, lane, row, v);
            const int64_t keep = key0 + row < kv_len ? 0 : (key0 + row - (kv_len - 1)) * 256;
            const char* src = (v ? vt : kt) + (off - keep);
            lds_dma16_flat(src, stage + 1024 * i);
        }
    }
}

// Issue this wave's loads of only the K half (kV = false) or only the V half
// of the tile at key0 (from `base`, the K or the V tensor) into `dst`, that
// half's own region of L::kKStage bytes; otherwise as stage_tile.
template <class L, int NW, bool kV>
__device__ __forceinline__ void stage_half(const StagePlan<L, NW>& p, const uint16_t* base, int64_t key0,
                                           int64_t kv_len, char* dst, int lane, int wave) {
    static_assert(L::kKLoads % NW == 0 && 2 * L::kKLoads == L::kLoads, "loads k < kN/2 fill K, the rest V");
    constexpr int kHalf = StagePlan<L, NW>::kN / 2;
    const char* tb = reinterpret_cast<const char*>(base + key0 * kHeadDim);
    if (key0 + kTile <= kv_len) {
#pragma unroll
        for (int k = kV ? kHalf : 0; k < (kV ? 2 * kHalf : kHalf); ++k) {
            const int i = wave + k * NW;
            lds_dma16(tb, p.off[k], dst + 1024 * (i - (kV ? L::kKLoads : 0)));
        }
    } else {
        for (int i = wave + (kV ? L::kKLoads : 0); i < (kV ? L::kLoads : L::kKLoads); i += NW) {
            int row;
            bool v;
            const uint32_t off = L::src(i, lane, row, v);
            const int64_t keep = key0 + row < kv_len ? 0 : (key0 + row - (kv_len - 1)) * 256;
            lds_dma16_flat(tb + (off - keep), dst + 1024 * (i - (kV ? L::kKLoads : 0)));
        }
    }
}

// Wait until at most N of this wave's vector-memory operations are pending.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait until at most one stage of this wave's direct loads is pending: the
// loads of the tile after the one being published may stay in flight.
template <class L, int NW>
__device__ __forceinline__ void wait_stage_loads(int wave) {
    if (wave < L::kLoads % NW)
        wait_vm<L::kLoads / NW + 1>();
    else
        wait_vm<L::kLoads / NW>();
}

// Combine a value with the one held by the lane 32 apart (the other half of
// the same MFMA column), with v_permlane32_swap: after the swap one copy holds
// the low half's value in every lane and the other the high half's, so every
// lane evaluates op(low, high) with the same operand order.
__device__ __forceinline__ void halves(float x, float& lo, float& hi) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    lo = __builtin_bit_cast(float, (unsigned)r[0]);
    hi = __builtin_bit_cast(float, (unsigned)r[1]);
}

// IEEE maximum (v_maximum_f32 / v_maximum3_f32): exact, and unlike fmaxf it
// needs no canonicalising moves in front of MFMA results.  The scores are
// finite or -inf, so it agrees with any other max.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Max of the 16 scores of one key block held by a lane, in four short chains
// of three-input maxima (the max is exact in any order).
__device__ __forceinline__ float block_max(const f32x16& s) {
    float c0 = vmax(vmax(s[0], s[1]), s[2]);
    float c1 = vmax(vmax(s[3], s[4]), s[5]);
    float c2 = vmax(vmax(s[6], s[7]), s[8]);
    float c3 = vmax(vmax(s[9], s[10]), s[11]);
    c0 = vmax(vmax(c0, s[12]), s[13]);
    c1 = vmax(vmax(c1, s[14]), s[15]);
    return vmax(vmax(c0, c1), vmax(c2, c3));
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    return z;
}

// ---------------------------------------------------------------------------
// One tile of the online softmax for the 32 query columns of a wave.
// Lane l owns query column j = l & 31; lane half h = l >> 5.
//   qf[st]  : B operand of k-step st: Q[query j][16st + 8h .. 16st + 8h + 7]
//   key0    : absolute index of the tile's first key
//   pos     : the column's position (keys > pos are masked) -- used when mask
//   mc, l   : running max in log2 units (max * c) and running sum
//   o[db]   : O^T accumulators for d rows 32*(dblk0+db) .. +31 of column j
// ---------------------------------------------------------------------------
// The reference max moves only when a tile's max exceeds it by more than
// kLazyTau (log2 units), so P <= 2^64 relative to the reference: a chunk's
// row sum is at most 2^74 and its accumulators 2^74 max|v|, and after the
// chunk fold a row's totals reach kv_len 2^64 and kv_len 2^64 max|v|, inside
// the fp32 range while kv_len max|v| < 2^64; relative rounding does not
// depend on the scale.  A high threshold makes the
// O rescale rare: on queries and keys with strong outlier channels (score
// spread of about 16 log2 units) a threshold of 8 rescales on about 2 tiles in
// 3, 32 on about 1 in 6 (mostly the first tile of a chunk, which skips it).
constexpr float kLazyTau = 64.0f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// o *= a.  o * 1 == o exactly, so skipping the multiply when no column of
// the wave moved its reference max leaves every bit as it is.
template <int NDB>
__device__ __forceinline__ void rescale_o(f32x16 (&o)[NDB], float a, bool any_grow) {
    if (any_grow) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int v = 0; v < 16; ++v) o[db][v] = o[db][v] * a;
        }
    }
}

// P of one 16-key step (kb, u): 8 exps and 4 paired converts to bf16.
__device__ __forceinline__ void p_only(const f32x16& s, int u, float c, float nmc, bf16x8& pf) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        f32x2 pp;
        pp[0] = exp2_hw(__builtin_fmaf(s[8 * u + e], c, nmc));
        pp[1] = exp2_hw(__builtin_fmaf(s[8 * u + e + 1], c, nmc));
        const bf16x2 pb = __builtin_convertvector(pp, bf16x2);
        pf[e] = pb[0];
        pf[e + 1] = pb[1];
    }
}

// The step's 4 dot2 row-sum terms (bf16 P pairs against (1, 1)) continue the
// lane's chain `acc`.
__device__ __forceinline__ void row_sum_dot2(const bf16x8& pf, float& acc) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const bf16x2 pb = {pf[e], pf[e + 1]};
        acc = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, acc, false);
    }
}

// P of one 16-key step with its row-sum terms.
__device__ __forceinline__ void p_step(const f32x16& s, int u, float c, float nmc, bf16x8& pf, float& acc) {
    p_only(s, u, c, nmc, pf);
    row_sum_dot2(pf, acc);
}

// o += P V for one 16-key step (kb, u) over the wave's NDB d blocks.
template <class L, int NDB>
__device__ __forceinline__ void pv_step(const bf16x8& pf, const char* sV, int kb, int u, int lane, f32x16 (&o)[NDB],
                                        int dblk0) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const bf16x8 vf = L::vt_frag(sV, kb, u, dblk0 + db, lane);
        o[db] = mfma(vf, pf, o[db]);
    }
}

// ---------------------------------------------------------------------------
// A tile in parts for the prefill, whose waves run one part while their SIMD
// partner runs the other: qk_fenced (the score products), then softmax_tile
// (mask, max, lazy reference update, P, rescale of o), then pv_fenced_rs
// (the P V products and the row sum) in the next product phase.
// ---------------------------------------------------------------------------
// Score products of one tile: block 0's chain, then block 1's, each fragment
// read four products ahead, the order fixed with scheduling fences (at most
// four fragments live).
template <class L>
__device__ __forceinline__ void qk_fenced(const bf16x8 (&qf)[8], const char* sK, int lane, f32x16& s0, f32x16& s1) {
    s0 = zero16();
    s1 = zero16();
    bf16x8 kf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) kf[i] = L::k_frag(sK, 0, i, lane);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        if (i < 8)
            s0 = mfma(kf[i & 3], qf[i & 7], s0);
        else
            s1 = mfma(kf[i & 3], qf[i & 7], s1);
        if (i + 4 < 16) kf[i & 3] = L::k_frag(sK, (i + 4) >> 3, (i + 4) & 7, lane);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// P V products of one tile in pv_step's order (key steps (0,0), (0,1), (1,0),
// (1,1), each over the d blocks), fragments read four products ahead behind
// scheduling fences, with the tile's row sum: after each key step's second
// product, that step's dot2 terms continue `acc` (in step order).  The dot2
// runs on the matrix pipe: beside this wave's own products it costs a few
// cycles, while beside the partner wave's products (in the softmax) it
// stalls them.
template <class L, int NDB>
__device__ __forceinline__ void pv_fenced_rs(const bf16x8 (&pf)[2][2], const char* sV, int lane, f32x16 (&o)[NDB],
                                             int dblk0, float& acc) {
    constexpr int N = 4 * NDB;
    constexpr int D = 4;
    bf16x8 vf[D];
#pragma unroll
    for (int i = 0; i < D; ++i) vf[i] = L::vt_frag(sV, (i / NDB) >> 1, (i / NDB) & 1, dblk0 + i % NDB, lane);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int step = i / NDB, db = i % NDB;
        o[db] = mfma(vf[i % D], pf[step >> 1][step & 1], o[db]);
        if (i + D < N) {
            const int sn = (i + D) / NDB, dn = (i + D) % NDB;
            vf[i % D] = L::vt_frag(sV, sn >> 1, sn & 1, dblk0 + dn, lane);
        }
        if (db == 1) row_sum_dot2(pf[step >> 1][step & 1], acc);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The softmax of a tile whose scores are in (s0, s1): mask (kMask: key j >
// pos gives -inf), tile max, lazy reference update, P (pf) and the rescale
// of o -- the rescale only when a column of the wave moved its reference (o *
// 1 == o), and none on a chunk's first tile (`first`: mc = -inf, l = 0, o =
// +0 on entry, so a = 0 and o * 0 = +0 = o).  The row sum comes later with
// the P V products (pv_fenced_rs); a_out is the factor the caller applies to
// l then: l = fma(l, a, sum).
template <int NDB, bool kMask>
__device__ __forceinline__ void softmax_tile(f32x16& s0, f32x16& s1, int lane, int64_t key0, int64_t pos, float c,
                                             float& mc, float& a_out, f32x16 (&o)[NDB], bf16x8 (&pf)[2][2],
                                             bool first) {
    if (kMask) {
        const int h = lane >> 5;
        const float ninf = -__builtin_inff();
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t kk = key0 + 8 * (v >> 2) + 4 * h + (v & 3);
            s0[v] = kk > pos ? ninf : s0[v];
            s1[v] = kk + 32 > pos ? ninf : s1[v];
        }
    }
    float mt = vmax(block_max(s0), block_max(s1));
    {
        float lo, hi;
        halves(mt, lo, hi);
        mt = vmax(lo, hi);
    }
    const float mtc = mt * c;
    const bool grow = (mtc - mc) > kLazyTau;
    const float mcn = grow ? mtc : mc;
    const bool any_grow = __builtin_amdgcn_ballot_w64(grow) != 0;
    // a = 1 for every column unless one of the wave's columns moved
    float a = 1.0f;
    if (any_grow) a = grow ? exp2_hw(mc - mcn) : 1.0f;
    const float nmc = -mcn;
    p_only(s0, 0, c, nmc, pf[0][0]);
    p_only(s0, 1, c, nmc, pf[0][1]);
    p_only(s1, 0, c, nmc, pf[1][0]);
    p_only(s1, 1, c, nmc, pf[1][1]);
    if (!first) rescale_o<NDB>(o, a, any_grow);
    a_out = a;
    mc = mcn;
}

// ---------------------------------------------------------------------------
// A tile in parts without branches, for the decode, which computes the
// scores of tile t + 1 beside the softmax and P V of tile t: qk_plain issues
// the score products (chains of both key blocks interleaved); softmax_flat
// does the mask, max, lazy reference update, P, row sum and rescale of o as
// softmax_tile does, but always computes a and always multiplies o by it (o *
// 1 == o exactly, so the bits are those of softmax_tile); pv_plain issues the
// P V products in pv_step's order.
// ---------------------------------------------------------------------------
template <class L>
__device__ __forceinline__ void qk_plain(const bf16x8 (&qf)[8], const char* sK, int lane, f32x16& s0, f32x16& s1) {
    s0 = zero16();
    s1 = zero16();
#pragma unroll
    for (int st = 0; st < 8; ++st) {
        s0 = mfma(L::k_frag(sK, 0, st, lane), qf[st], s0);
        s1 = mfma(L::k_frag(sK, 1, st, lane), qf[st], s1);
    }
}

template <int NDB, bool kMask>
__device__ __forceinline__ void softmax_flat(f32x16& s0, f32x16& s1, int lane, int64_t key0, int64_t pos, float c,
                                             float& mc, float& l, f32x16 (&o)[NDB], bf16x8 (&pf)[2][2]) {
    if (kMask) {
        const int h = lane >> 5;
        const float ninf = -__builtin_inff();
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t kk = key0 + 8 * (v >> 2) + 4 * h + (v & 3);
            s0[v] = kk > pos ? ninf : s0[v];
            s1[v] = kk + 32 > pos ? ninf : s1[v];
        }
    }
    float mt = vmax(block_max(s0), block_max(s1));
    {
        float lo, hi;
        halves(mt, lo, hi);
        mt = vmax(lo, hi);
    }
    const float mtc = mt * c;
    const bool grow = (mtc - mc) > kLazyTau;
    const float mcn = grow ? mtc : mc;
    const float a = grow ? exp2_hw(mc - mcn) : 1.0f;
    const float nmc = -mcn;
    float acc = 0.0f;  // this lane's row-sum chain over the tile's 16 dot2 terms
    p_step(s0, 0, c, nmc, pf[0][0], acc);
    p_step(s0, 1, c, nmc, pf[0][1], acc);
    p_step(s1, 0, c, nmc, pf[1][0], acc);
    p_step(s1, 1, c, nmc, pf[1][1], acc);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int v = 0; v < 16; ++v) o[db][v] = o[db][v] * a;
    }
    float ls_lo, ls_hi;
    halves(acc, ls_lo, ls_hi);
    l = __builtin_fmaf(l, a, ls_lo + ls_hi);
    mc = mcn;
}

template <class L, int NDB>
__device__ __forceinline__ void pv_plain(const bf16x8 (&pf)[2][2], const char* sV, int lane, f32x16 (&o)[NDB],
                                         int dblk0) {
    pv_step<L, NDB>(pf[0][0], sV, 0, 0, lane, o, dblk0);
    pv_step<L, NDB>(pf[0][1], sV, 0, 1, lane, o, dblk0);
    pv_step<L, NDB>(pf[1][0], sV, 1, 0, lane, o, dblk0);
    pv_step<L, NDB>(pf[1][1], sV, 1, 1, lane, o, dblk0);
}

// Fold weights of one chunk into the running total (scalars of one column,
// maxima in log2 units).
__device__ __forceinline__ void fold_scalars(float Mc, float mc, float& Mcn, float& A, float& B) {
    Mcn = fmaxf(Mc, mc);
    A = (Mcn == Mc) ? 1.0f : exp2_hw(Mc - Mcn);
    B = (Mcn == mc) ? 1.0f : exp2_hw(mc - Mcn);
}

__device__ __forceinline__ float fold_value(float O, float A, float o, float B) {
    return __builtin_fmaf(O, A, o * B);
}

// out = bf16_rne(q) with q = O / L by Markstein's reciprocal-and-correction
// sequence: y = rcp(L) refined by one Newton step, q0 = O y, r = O - q0 L
// (exact, one fma), q = q0 + r y.  It costs a few instructions instead of a
// full IEEE division per element (y is the same for a row, so it is computed
// once); every kernel uses this same sequence.  L >= 1 (the key that set the
// reference max contributes 2^0), so no step meets a denormal or infinity.
__device__ __forceinline__ uint16_t finalize(float O, float L) {
    float y = __builtin_amdgcn_rcpf(L);
    y = __builtin_fmaf(__builtin_fmaf(-L, y, 1.0f), y, y);
    const float q0 = O * y;
    const float r = __builtin_fmaf(-q0, L, O);
    const __bf16 q = (__bf16)__builtin_fmaf(r, y, q0);
    return __builtin_bit_cast(uint16_t, q);
}

// Natural-log log-sum-exp of a row from its final (Mc, L): Mc + log2(L) is
// log2 of sum_j 2^(c s_j) = log2 of sum_j exp(scale s_j).  L >= 1 (the key
// that set the reference max contributes 2^0 or more), so v_log_f32 sees no
// denormal.
__device__ __forceinline__ float lse_of(float Mc, float L) {
    return (Mc + __builtin_amdgcn_logf(L)) * 0.693147182f;
}

}  // namespace kb
