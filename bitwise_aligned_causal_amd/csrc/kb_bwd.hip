// kb_bwd: deterministic backward of the causal GQA attention for gfx950.
//
// The pages cover the forward only (KernelBraid / AReaL-TIK README,
// "Features": the release covers forward attention; "Background": training
// forward and backward still run).  This is the gradient of that forward for
// full causal sequences, recomputing P from the log-sum-exp the forward
// returns (the usual flash-attention recomputation), with every output
// element reduced in one fixed order -- no atomics -- so its bits depend only
// on the inputs:
//
//   bwd_prep_kernel  D_i = <dO_i, O_i> and lse2_i = lse_i * log2(e) per row
//   bwd_dkdv_kernel  one wave per 32 keys of a KV head (256 keys, 8 waves
//                    per workgroup; the block's V rows stay in LDS); the
//                    Q / dO rows of the 4 query heads stream through LDS in
//                    32-row tiles, and each wave computes for its keys
//                      S    = Q K^T           (A = Q rows,  B = K rows in registers)
//                      dP   = dO V^T          (A = dO rows, B = V rows from LDS)
//                      P    = exp2(S c - lse2),  dS = P (dP - D)
//                      dV^T += dO^T P,  dK^T += Q^T dS
//                    (the last two with their first operands read
//                    transposed from LDS)
//   bwd_dq_kernel    one wave per 32 query rows; K / V tiles of 64 keys stream
//                    through LDS as in the forward:
//                      S^T  = K Q^T,  dP^T = V dO^T,  dQ^T += K^T dS^T
// All products are v_mfma_f32_32x32x16_bf16 with fp32 accumulation; P and dS
// are rounded to bf16 (RNE) as the operands of the second products.  Both
// kernels run their two wave groups in ping-pong, as the forward prefill does:
// one wave of a SIMD multiplies while its partner computes P and dS.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <initializer_list>

#include "../../include/kb_attn.h"
#include "kb_contract.h"

namespace kb {
namespace bwd {

// ---------------------------------------------------------------------------
// LDS tiles: rows of 272 bytes (256 of data, 16 of padding that nothing
// reads), the tile's row r stored at tile row
//   prow(r) = 16 (r >> 4) + 4 (r & 3) + ((r >> 2) & 3)
// (the two 2-bit fields of r swapped within each group of 16 rows, so prow
// is its own inverse).  The row stride is 16 bytes past a multiple of 256,
// so tile row t starts at bank group t mod 16:
//   row reads (16 lanes: 16 consecutive rows, one 16-byte chunk) meet 16
//     distinct tile rows mod 16, hence 16 distinct bank groups;
//   transposing reads (32 lanes: the 4 rows 4m .. 4m + 3, 64 bytes each)
//     meet tile rows 4n + (m mod 4), whose starts lie 64 bytes apart.
// Every fragment address is a per-lane base plus an immediate offset.
// ---------------------------------------------------------------------------
constexpr int kRowBytes = 272;

__device__ __forceinline__ int prow(int r) { return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3); }

// A tile of R rows: R * 17 slots of 16 bytes filled by whole one-KiB direct
// loads (the last load of a 32-row tile runs into the tile's spare bytes).
template <int R>
struct PermTile {
    static constexpr int kLoads = (R * 17 + 63) / 64;
    static constexpr int kBytes = kLoads * 1024;
};

// Source byte offset, from the tile's first row, of direct load i, lane
// `lane`: slot 64 i + lane is chunk c of tile row t, i.e. chunk min(c, 15) of
// row prow(t).  Rows beyond min(last, R - 1) read that row instead (they are
// masked or weighted by zero later; the padding chunk is never read).
template <int R>
__device__ __forceinline__ uint32_t perm_src(int i, int lane, int64_t last) {
    const int p = 64 * i + lane;
    const int t = p / 17, c = p - 17 * t;
    const int64_t lim = last < R - 1 ? last : R - 1;
    const int64_t r = prow(t) < lim ? prow(t) : lim;
    return (uint32_t)(r * 256 + (c < 16 ? c : 15) * 16);
}

// A planned offset (for a tile whose rows all lie inside the sequence)
// re-aimed at row `last` when its row lies beyond it: the row is off >> 8 and
// the chunk offset off & 255.
__device__ __forceinline__ uint32_t clamp_src(uint32_t off, int64_t last) {
    const int64_t r = off >> 8;
    return r > last ? (uint32_t)(last * 256) + (off & 255u) : off;
}

// lds_dma16 with the scalar base forced into scalar registers: the base is
// uniform by construction, but the compiler cannot always prove it.
__device__ __forceinline__ void dma16(const char* base, uint32_t voff, char* dst) {
    const uint64_t p = (uint64_t)(uintptr_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    lds_dma16(reinterpret_cast<const char*>((uintptr_t)(((uint64_t)hi << 32) | lo)), voff, dst);
}

// The LDS byte address of a pointer into a __shared__ array (the low 32 bits
// of its generic address), as an LDS pointer: fragment addresses built on it
// keep their constant parts as instruction offsets.
typedef __attribute__((address_space(3))) const char lds_byte;
__device__ __forceinline__ lds_byte* to_lds(const char* p) {
    return (lds_byte*)(uintptr_t)(uint32_t)(uintptr_t)p;
}

// Row fragment: lane (row 32 blk + (lane & 31), half h) holds bf16
// [16 st + 8h, 16 st + 8h + 7] of its row -- the A operand of a product whose
// rows are the tile's rows, or the B operand whose columns are.  `rb` is
// row_base(lane) (prow(32 blk + i) = 32 blk + prow(i)).
__device__ __forceinline__ int row_base(int lane) { return prow(lane & 31) * kRowBytes + (lane >> 5) * 16; }
__device__ __forceinline__ bf16x8 row_frag(const char* tile, int rb, int blk, int st) {
    const lds_byte* p = to_lds(tile) + rb + blk * 32 * kRowBytes + st * 32;
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p));
}

// Transposed fragment: the A operand X^T[d][rows] for d block dblk and the
// 16-row step (blk, u) of the tile, with the row order of an MFMA result
// column: lane (d = 32 dblk + j, half h) holds, in slot order,
//   X[R0 + 4h + {0..3}][d], X[R0 + 8 + 4h + {0..3}][d],   R0 = 32 blk + 16 u
// (two ds_read_b64_tr_b16).  Lane (g = lane >> 4, n = (lane >> 2) & 3,
// jj = lane & 3) points at row R0 + 4 (g >> 1) + n, tile row
// R0 + 4n + (g >> 1), and d = 32 dblk + 16 (g & 1) + 4 jj; the second read is
// 8 rows on, 2 tile rows on.  `tb` is tr_base(lane).
__device__ __forceinline__ int tr_base(int lane) {
    const int g = lane >> 4, n = (lane >> 2) & 3, jj = lane & 3;
    return (4 * n + (g >> 1)) * kRowBytes + 32 * (g & 1) + 8 * jj;
}
__device__ __forceinline__ bf16x8 tr_frag(const char* tile, int tb, int blk, int u, int dblk) {
    const lds_byte* p0 = to_lds(tile) + tb + (32 * blk + 16 * u) * kRowBytes + 64 * dblk;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 2 * kRowBytes));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 all = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, all);
}

// bf16 (RNE) of elements 8u .. 8u + 7 of an MFMA result: the k-slots of the
// 16-row step u in the order tr_frag reads the other operand.
__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int u) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        f32x2 pp;
        pp[0] = x[8 * u + e];
        pp[1] = x[8 * u + e + 1];
        const bf16x2 pb = __builtin_convertvector(pp, bf16x2);
        r[e] = pb[0];
        r[e + 1] = pb[1];
    }
    return r;
}

// Stores 16 fp32 of an MFMA result column, times `mul`, as bf16 into row
// `dst` (128 elements): element v holds d = 32 dblk + 8 (v >> 2) + 4h + (v & 3).
__device__ __forceinline__ void store_col(uint16_t* dst, const f32x16 (&acc)[4], float mul, int h) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
            uint32_t e[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const __bf16 x = (__bf16)(acc[db][4 * b4 + i] * mul);
                e[i] = __builtin_bit_cast(uint16_t, x);
            }
            uint2 packed;
            packed.x = e[0] | (e[1] << 16);
            packed.y = e[2] | (e[3] << 16);
            *reinterpret_cast<uint2*>(dst + 32 * db + 8 * b4 + 4 * h) = packed;
        }
    }
}

constexpr float kLog2e = 1.44269502f;  // fp32(log2 e)

struct BwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* o;
    const uint16_t* dout;
    const float* lse;
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    float* ws_d;     // [batch * Hq, s_pad]  D_i
    float* ws_lse2;  // [batch * Hq, s_pad]  lse_i * log2 e
    int64_t seq_len, s_pad;
    int32_t batch, n_kv_heads;
    float c;      // fp32(scale * log2 e), as in the forward
    float scale;  // fp32 scale
};

// Where one sequence's rows live.  Query head h (0 .. Hq - 1 of the sequence)
// row i is row h * hstride + q_row0 + i of q, o, dout, dq (and of lse);
// KV head g key j is row g * hstride + kv_row0 + j of k, v, dk, dv; its
// D / lse2 entries are at h * ws_hstride + ws_row0 + i.  Dense batches:
// q_row0 = b Hq S, kv_row0 = b Hkv S, hstride = S, ws_row0 = b Hq S_pad,
// ws_hstride = S_pad.  Packed ragged batches [H, T, 128]: q_row0 = kv_row0 =
// the sequence's first packed row, hstride = T, ws_row0 = its first padded
// row, ws_hstride = T_pad.
struct BwdSeq {
    int64_t S;
    int64_t q_row0, kv_row0, hstride;
    int64_t ws_row0, ws_hstride;
};

__device__ __forceinline__ BwdSeq dense_seq(const BwdArgs& a, int b) {
    const int64_t hq = (int64_t)kGroup * a.n_kv_heads;
    BwdSeq sq;
    sq.S = a.seq_len;
    sq.q_row0 = (int64_t)b * hq * a.seq_len;
    sq.kv_row0 = (int64_t)b * a.n_kv_heads * a.seq_len;
    sq.hstride = a.seq_len;
    sq.ws_row0 = (int64_t)b * hq * a.s_pad;
    sq.ws_hstride = a.s_pad;
    return sq;
}

// Ragged launches: at most kBwdMaxSeqs sequences, each padded to a multiple
// of 64 rows in the workspace; unit_kv / unit_dq are the prefix sums of the
// dK/dV and dQ work units (KV heads x 256-key blocks, KV heads x 64-row
// blocks) of the sequences in this launch.
constexpr int kBwdMaxSeqs = 64;
struct BwdTable {
    int64_t row0[kBwdMaxSeqs];  // first packed row
    int64_t pad0[kBwdMaxSeqs];  // first padded workspace row
    int32_t len[kBwdMaxSeqs];
    int32_t unit_kv[kBwdMaxSeqs + 1];
    int32_t unit_dq[kBwdMaxSeqs + 1];
    int32_t n_seqs;
    int64_t t_rows, t_pad;     // rows per head of the packed tensors and of the padded workspace
    int64_t p_begin, p_count;  // the launch's sequences' padded rows (consecutive)
};

__device__ __forceinline__ BwdSeq table_seq(const BwdTable& t, int s) {
    BwdSeq sq;
    sq.S = t.len[s];
    sq.q_row0 = t.row0[s];
    sq.kv_row0 = t.row0[s];
    sq.hstride = t.t_rows;
    sq.ws_row0 = t.pad0[s];
    sq.ws_hstride = t.t_pad;
    return sq;
}

// ---------------------------------------------------------------------------
// D and lse2 per row: 8 lanes per row, 16 elements per lane in order, then a
// fixed xor butterfly over the 8 lanes.  Padding rows (i >= the sequence's
// length) get 0.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void prep_row(const BwdArgs& a, int64_t src_row, int64_t ws_row, bool valid,
                                         bool in_range, int part) {
    float acc = 0.0f;
    if (valid) {
        const int64_t src = src_row * kHeadDim + 16 * part;
        const u32x4* dp = reinterpret_cast<const u32x4*>(a.dout + src);
        const u32x4* op = reinterpret_cast<const u32x4*>(a.o + src);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const bf16x8 x = __builtin_bit_cast(bf16x8, dp[half]);
            const bf16x8 y = __builtin_bit_cast(bf16x8, op[half]);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)x[e], (float)y[e], acc);
        }
    }
    acc = acc + __shfl_xor(acc, 1);
    acc = acc + __shfl_xor(acc, 2);
    acc = acc + __shfl_xor(acc, 4);
    if (in_range && part == 0) {
        a.ws_d[ws_row] = valid ? acc : 0.0f;
        a.ws_lse2[ws_row] = valid ? a.lse[src_row] * kLog2e : 0.0f;
    }
}

// dense: workspace row w = (b Hq + h) S_pad + i
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
    const int64_t row = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
    const int64_t n_rows = (int64_t)a.batch * kGroup * a.n_kv_heads * a.s_pad;
    const bool in_range = row < n_rows;
    const int64_t bh = in_range ? row / a.s_pad : 0;
    const int64_t i = in_range ? row % a.s_pad : 0;
    prep_row(a, bh * a.seq_len + i, row, in_range && i < a.seq_len, in_range, threadIdx.x & 7);
}

// ragged: block x covers padded rows p_begin + 32 (x % nb) .. + 31 of query
// head x / nb, nb = p_count / 32 blocks per head; a block never straddles
// two sequences (each is padded to a multiple of 64 rows)
__global__ __launch_bounds__(256) void bwd_prep_varlen_kernel(BwdArgs a, BwdTable t) {
    const int64_t nb = t.p_count / 32;
    const int64_t h = blockIdx.x / nb;
    const int64_t p = t.p_begin + (blockIdx.x % nb) * 32 + (threadIdx.x >> 3);  // padded row
    int s = 0;
    while (s + 1 < t.n_seqs && t.pad0[s + 1] <= p) ++s;
    const int64_t i = p - t.pad0[s];
    const bool in_range = p < t.pad0[s] + ((t.len[s] + 63) / 64) * 64 && p >= t.pad0[s];
    prep_row(a, h * t.t_rows + t.row0[s] + i, h * t.t_pad + p, in_range && i < t.len[s], in_range,
             threadIdx.x & 7);
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup = 8 waves on 256 keys [K0, K0 + 256) of one (sequence,
// KV head).  Wave w owns keys k0 = K0 + 32 w .. + 31: it holds their K and V
// rows as B operands and their dK^T and dV^T accumulators, and per work item
// (32 query rows q0 .. q0 + 31 of one query head) computes
//   S  = Q K^T,  dP = dO V^T                (A = Q / dO rows from LDS)
//   P  = exp2(S c - lse2), masked on edge tiles;  dS = P (dP - D)
//   dV^T += dO^T P,  dK^T += Q^T dS         (A = dO^T / Q^T from LDS)
// Work items t = 0, 1, ...: query tile q0 = qlast - 32 (t / 4) of query head
// 4g + (t % 4), from the last tile qlast down to K0; a wave skips the items
// whose rows all precede its keys.  A 4-stage LDS ring holds each item's Q
// and dO rows and its 32 lse2 and 32 D values, loaded two items ahead (an
// item is read in two product phases of each wave group, see dkdv_body).
// dK^T and dV^T accumulate over the items in that fixed order.
// ---------------------------------------------------------------------------
constexpr int kKvWaves = 8;
constexpr int kKvKeys = 32 * kKvWaves;
constexpr int kQTileBytes = PermTile<32>::kBytes;     // 9 KiB
constexpr int kKvTileLoads = PermTile<32>::kLoads;    // 9
constexpr int kKvStageBytes = 2 * kQTileBytes + 256;  // Q, dO, lse2[32], D[32]
constexpr int kKvStages = 4;
// the workgroup's 256 V rows stay in LDS (a permuted padded tile) after the ring
constexpr int kKvVBytes = PermTile<kKvKeys>::kBytes;  // 68 KiB
constexpr int kKvVLoads = PermTile<kKvKeys>::kLoads;  // 68
// a stage is 2 x 9 tile loads and two loads of 32 floats (lse2, D); wave w
// issues loads w, w + 8, w + 16: waves 0..3 three per stage, waves 4..7 two
constexpr int kKvStageLoads = 2 * kKvTileLoads + 2;
constexpr int kKvLoadsMax = (kKvStageLoads + kKvWaves - 1) / kKvWaves;

// Per-lane source offsets of this wave's tile loads for a tile whose 32 rows
// all lie inside the sequence.
struct KvPlan {
    uint32_t o[kKvLoadsMax];
    __device__ uint32_t off(int k) const { return o[k]; }
};

__device__ __forceinline__ void kv_stage(const BwdArgs& a, const BwdSeq& sq, int g, int t, int64_t qlast,
                                         const KvPlan& plan, char* stage, int w, int lane) {
    const int64_t q0 = qlast - 32 * (t >> 2);
    const int64_t hh = kGroup * g + (t & 3);  // query head of the item
    const int64_t qrow = hh * sq.hstride + sq.q_row0 + q0;
    const char* qb = reinterpret_cast<const char*>(a.q + qrow * kHeadDim);
    const char* db = reinterpret_cast<const char*>(a.dout + qrow * kHeadDim);
    const int64_t last = sq.S - 1 - q0;  // last valid row, relative to q0
#pragma unroll
    for (int k = 0; k < kKvLoadsMax; ++k) {
        const int i = w + kKvWaves * k;
        if (i >= kKvStageLoads) break;
        if (i < 2 * kKvTileLoads) {
            const bool dO = i >= kKvTileLoads;
            const int ti = dO ? i - kKvTileLoads : i;
            const uint32_t o = plan.off(k);
            const uint32_t off = last >= 31 ? o : clamp_src(o, last);
            dma16(dO ? db : qb, off, stage + (dO ? kQTileBytes : 0) + 1024 * ti);
        } else if (lane < 8) {
            // lse2 (load 18) or D (load 19) of the 32 rows, 16 bytes a lane;
            // padded arrays, in bounds
            const bool dl = i > 2 * kKvTileLoads;
            const float* src = (dl ? a.ws_d : a.ws_lse2) + hh * sq.ws_hstride + sq.ws_row0 + q0;
            dma16(reinterpret_cast<const char*>(src), (uint32_t)(16 * lane), stage + 2 * kQTileBytes + (dl ? 128 : 0));
        }
    }
}

// One work item of a wave, in three parts (the ping-pong below runs the
// first and last on the matrix pipe and the middle one on the vector ALU).
// kv_first: S = Q K^T and dP = dO V^T side by side, the Q, dO and V
// fragments read one step ahead of their products (scheduling fences keep
// this order: left alone, the compiler reads every fragment first and runs
// out of registers; two steps ahead spills in the ping-pong).
__device__ __forceinline__ void kv_first(const bf16x8 (&kf)[8], const char* sVw, const char* sQ, const char* sD,
                                         int rb, f32x16& s, f32x16& dp) {
    s = zero16();
    dp = zero16();
    bf16x8 aq[2], ad[2], bv[2];
    aq[0] = row_frag(sQ, rb, 0, 0);
    ad[0] = row_frag(sD, rb, 0, 0);
    bv[0] = row_frag(sVw, rb, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
        if (st + 1 < 8) bv[(st + 1) % 2] = row_frag(sVw, rb, 0, st + 1);
        if (st + 1 < 8) aq[(st + 1) % 2] = row_frag(sQ, rb, 0, st + 1);
        s = mfma(aq[st % 2], kf[st], s);
        if (st + 1 < 8) ad[(st + 1) % 2] = row_frag(sD, rb, 0, st + 1);
        dp = mfma(ad[st % 2], bv[st % 2], dp);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// kv_vector: P and dS in bf16 (pb, sb).  Element v of an MFMA result: query
// q0 + 8 (v >> 2) + 4h + (v & 3), key k0 + j; on an edge tile it counts when
// k0 + j <= query < S, i.e. lo <= 8 (v >> 2) + (v & 3) < hi.  The mask is a
// uniform branch around the selects only, so the accumulators never cross a
// join.
__device__ __forceinline__ void kv_vector(f32x16& s, f32x16& dp, const float* sL, int lane, float c, bool edge,
                                          int lo, int hi, bf16x8 (&pb)[2], bf16x8 (&sb)[2]) {
    const int h = lane >> 5;
#pragma unroll
    for (int b4 = 0; b4 < 4; ++b4) {
        const float4 l2 = *reinterpret_cast<const float4*>(sL + 8 * b4 + 4 * h);
        const float lv[4] = {l2.x, l2.y, l2.z, l2.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) s[4 * b4 + i] = exp2_hw(__builtin_fmaf(s[4 * b4 + i], c, -lv[i]));
    }
    if (edge) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int off = 8 * (v >> 2) + (v & 3);
            s[v] = (lo <= off && off < hi) ? s[v] : 0.0f;
        }
    }
#pragma unroll
    for (int b4 = 0; b4 < 4; ++b4) {
        const float4 d4 = *reinterpret_cast<const float4*>(sL + 32 + 8 * b4 + 4 * h);
        const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) dp[4 * b4 + i] = s[4 * b4 + i] * (dp[4 * b4 + i] - dv[i]);
    }
    pb[0] = pack8(s, 0);
    pb[1] = pack8(s, 1);
    sb[0] = pack8(dp, 0);
    sb[1] = pack8(dp, 1);
}

// kv_second: dV^T += dO^T P and dK^T += Q^T dS, the transposed fragments read
// one step ahead.
__device__ __forceinline__ void kv_second(const char* sQ, const char* sD, int tb, const bf16x8 (&pb)[2],
                                          const bf16x8 (&sb)[2], f32x16 (&acck)[4], f32x16 (&accv)[4]) {
    bf16x8 td = tr_frag(sD, tb, 0, 0, 0), tq = tr_frag(sQ, tb, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int x = 0; x < 8; ++x) {
        const int u = x >> 2, db = x & 3;
        bf16x8 nd, nq;
        if (x + 1 < 8) nd = tr_frag(sD, tb, 0, (x + 1) >> 2, (x + 1) & 3);
        accv[db] = mfma(td, pb[u], accv[db]);
        if (x + 1 < 8) nq = tr_frag(sQ, tb, 0, (x + 1) >> 2, (x + 1) & 3);
        acck[db] = mfma(tq, sb[u], acck[db]);
        __builtin_amdgcn_sched_barrier(0);
        if (x + 1 < 8) {
            td = nd;
            tq = nq;
        }
    }
}

// One dK/dV workgroup: keys [256 kb, 256 kb + 256) of KV head g of one sequence.
__device__ __forceinline__ void dkdv_body(const BwdArgs& a, const BwdSeq& sq, int g, int kb, char* smem) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31, h = lane >> 5;
    const int64_t S = sq.S;
    const int64_t K0 = (int64_t)kb * kKvKeys;
    const int64_t k0 = K0 + 32 * w;  // this wave's first key
    // query tiles from the last one down to K0: every block of a (sequence,
    // KV head) starts at the same rows, so the blocks running together on an
    // XCD read the same Q / dO rows at about the same time (one L2 fetch)
    const int64_t qlast = ((S - 1) >> 5) << 5;
    const int n_items = 4 * (int)((qlast - K0) / 32 + 1);
    const int rb = row_base(lane), tb = tr_base(lane);
    KvPlan plan;
#pragma unroll
    for (int k = 0; k < kKvLoadsMax; ++k) {
        const int i = w + kKvWaves * k;
        const int ti = i < kKvTileLoads ? i : i - kKvTileLoads;
        plan.o[k] = i < 2 * kKvTileLoads ? perm_src<32>(ti, lane, 31) : 0u;
    }

    const int64_t kv0 = (int64_t)g * sq.hstride + sq.kv_row0;  // row of key 0
    char* sV = smem + kKvStages * kKvStageBytes;
    {
        // the block's V rows (rows beyond S read row S - 1)
        const char* vb = reinterpret_cast<const char*>(a.v + (kv0 + K0) * kHeadDim);
        for (int i = w; i < kKvVLoads; i += kKvWaves)
            dma16(vb, perm_src<kKvKeys>(i, lane, S - 1 - K0), sV + 1024 * i);
    }
    kv_stage(a, sq, g, 0, qlast, plan, smem, w, lane);
    if (n_items >= 2) kv_stage(a, sq, g, 1, qlast, plan, smem + kKvStageBytes, w, lane);

    // this wave's K rows as B operands: lane (key j, half h) holds row k0 + j,
    // d = 16 st + 8h .. + 7 (rows beyond S read row S - 1)
    bf16x8 kf[8];
    {
        int64_t key = k0 + j;
        key = key < S ? key : S - 1;
        const uint16_t* ks = a.k + (kv0 + key) * kHeadDim;
#pragma unroll
        for (int st = 0; st < 8; ++st)
            kf[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ks + 16 * st + 8 * h));
    }
    // the fragments are complete before the item loop: otherwise the compiler
    // keeps waits for them inside the loop, where they also hold each item
    // behind the direct loads it has just issued
    wait_vm<0>();

    f32x16 acck[4], accv[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        acck[db] = zero16();
        accv[db] = zero16();
    }
    const float c = a.c;
    const int grp = w >> 2;
    // Ping-pong, as in the forward prefill: waves w and w + 4 share a SIMD;
    // group 0 runs item t as products (the second products of item t - 1,
    // then the first of item t) followed by the vector work of item t, group
    // 1 the same one step behind.  One barrier per item, before the products
    // of item t, after every wave has waited for its own loads of t; the
    // loads of item t + 2 are issued at the start of the vector work of item
    // t, into the stage of item t - 2 (last read in the products of t - 1).
    // A wave skips the items whose rows all precede its keys (a suffix of
    // the item order), but issues their loads and meets every barrier.
    auto tile_start = [&](int t) {
        if (t < n_items) {
            if (t + 1 < n_items && grp == 0) {
                if (w < kKvStageLoads - (kKvLoadsMax - 1) * kKvWaves)
                    wait_vm<kKvLoadsMax>();
                else
                    wait_vm<kKvLoadsMax - 1>();
            } else {
                wait_vm<0>();
            }
        }
        __syncthreads();
    };
    auto item_live = [&](int t) { return qlast - 32 * (t >> 2) >= k0; };
    f32x16 s, dp;
    bf16x8 pb[2], sb[2];
    auto products = [&](int t) {
        __builtin_amdgcn_s_setprio(3);
        if (t >= 1 && item_live(t - 1)) {
            const char* stage = smem + ((t - 1) % kKvStages) * kKvStageBytes;
            kv_second(stage, stage + kQTileBytes, tb, pb, sb, acck, accv);
        }
        if (t < n_items && item_live(t)) {
            const char* stage = smem + (t % kKvStages) * kKvStageBytes;
            kv_first(kf, sV + 32 * w * kRowBytes, stage, stage + kQTileBytes, rb, s, dp);
        }
    };
    auto vector_work = [&](int t) {
        __builtin_amdgcn_s_setprio(0);
        if (t + 2 < n_items)
            kv_stage(a, sq, g, t + 2, qlast, plan, smem + ((t + 2) % kKvStages) * kKvStageBytes, w, lane);
        if (item_live(t)) {
            const int64_t q0 = qlast - 32 * (t >> 2);
            const char* stage = smem + (t % kKvStages) * kKvStageBytes;
            const bool edge = q0 == k0 || q0 + 32 > S;
            const int lo = (int)(k0 - q0) + j - 4 * h;
            const int hi = (int)(S - q0 < 64 ? S - q0 : 64) - 4 * h;
            kv_vector(s, dp, reinterpret_cast<const float*>(stage + 2 * kQTileBytes), lane, c, edge, lo, hi, pb, sb);
        }
    };
    if (grp == 0) {
        for (int t = 0; t < n_items; ++t) {
            tile_start(t);
            products(t);
            vector_work(t);
        }
        tile_start(n_items);
        products(n_items);
    } else {
        tile_start(0);
        products(0);
        for (int t = 0; t < n_items; ++t) {
            tile_start(t + 1);
            vector_work(t);
            products(t + 1);
        }
    }
    __builtin_amdgcn_s_setprio(0);
    const int64_t row = (kv0 + k0 + j) * kHeadDim;
    if (k0 + j < S) {
        store_col(a.dv + row, accv, 1.0f, h);
        store_col(a.dk + row, acck, a.scale, h);
    }
}

// Dense batch: [B, H, S, 128].
__global__ __launch_bounds__(64 * kKvWaves) void bwd_dkdv_kernel(BwdArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[kKvStages * kKvStageBytes + kKvVBytes];
    const int n_kb = (int)((a.seq_len + kKvKeys - 1) / kKvKeys);
    const int nbg = a.batch * a.n_kv_heads;
    const int x = blockIdx.x;
    int bg, kb;
    if ((nbg & 7) == 0) {
        // XCD k (x % 8) takes the (b, g) pairs k, k + 8, ..., each pair's key
        // blocks longest work first
        const int i = x >> 3;
        bg = (i / n_kb) * 8 + (x & 7);
        kb = i % n_kb;
    } else {
        bg = x % nbg;
        kb = x / nbg;
    }
    dkdv_body(a, dense_seq(a, bg / a.n_kv_heads), bg % a.n_kv_heads, kb, smem);
}

// Ragged batch (packed [H, T, 128]): units of a sequence are (256-key block,
// KV head), longest blocks first.
__global__ __launch_bounds__(64 * kKvWaves) void bwd_dkdv_varlen_kernel(BwdArgs a, BwdTable t) {
    __shared__ __attribute__((aligned(1024))) char smem[kKvStages * kKvStageBytes + kKvVBytes];
    const int x = blockIdx.x;
    int s = 0;
    while (s + 1 < t.n_seqs && t.unit_kv[s + 1] <= x) ++s;
    const int u = x - t.unit_kv[s];
    dkdv_body(a, table_seq(t, s), u % a.n_kv_heads, u / a.n_kv_heads, smem);
}

// ---------------------------------------------------------------------------
// dQ: workgroup = 8 waves = the 4 query heads of one KV head x 2 halves of
// the 64 positions [64 pb, 64 pb + 64), as in the forward; K / V tiles of 64
// keys (K and V, permuted padded tiles) stream through a 4-stage ring, loads two
// tiles ahead.  Wave column j is query row 64 pb + 32 (w >> 2) + j.
// ---------------------------------------------------------------------------
constexpr int kDqWaves = 8;
constexpr int kDqStages = 4;
constexpr int kDqTileLoads = PermTile<64>::kLoads;  // 17
constexpr int kDqTileBytes = PermTile<64>::kBytes;  // 17 KiB
constexpr int kDqStageBytes = 2 * kDqTileBytes;     // K, V
// a stage is 2 x 17 loads; wave w issues loads w, w + 8, ...: waves 0, 1
// five per stage, waves 2..7 four
constexpr int kDqStageLoads = 2 * kDqTileLoads;
constexpr int kDqLoadsMax = (kDqStageLoads + kDqWaves - 1) / kDqWaves;

// Per-lane source offsets of this wave's loads for a tile whose 64 keys all
// lie inside the sequence.
struct DqPlan {
    uint32_t off[kDqLoadsMax];
};

__device__ __forceinline__ void dq_stage(const uint16_t* kb, const uint16_t* vb, int64_t key0, int64_t S,
                                         const DqPlan& plan, char* stage, int w) {
    const char* kt = reinterpret_cast<const char*>(kb + key0 * kHeadDim);
    const char* vt = reinterpret_cast<const char*>(vb + key0 * kHeadDim);
    const int64_t last = S - 1 - key0;  // last valid key, relative to key0
#pragma unroll
    for (int k = 0; k < kDqLoadsMax; ++k) {
        const int i = w + kDqWaves * k;
        if (i >= kDqStageLoads) break;
        const bool vtile = i >= kDqTileLoads;
        const int ti = vtile ? i - kDqTileLoads : i;
        const uint32_t off = last >= 63 ? plan.off[k] : clamp_src(plan.off[k], last);
        dma16(vtile ? vt : kt, off, stage + (vtile ? kDqTileBytes : 0) + 1024 * ti);
    }
}

// One dQ workgroup: positions [64 pb, 64 pb + 64) of the 4 query heads of KV
// head g of one sequence.
__device__ __forceinline__ void dq_body(const BwdArgs& a, const BwdSeq& sq, int g, int pb, char* smem) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31, h = lane >> 5;

    const int64_t S = sq.S;
    const int64_t hh = kGroup * g + (w & 3);  // this wave's query head
    const int64_t pos = (int64_t)pb * 64 + 32 * (w >> 2) + j;
    const bool active = pos < S;
    const int64_t qrow0 = hh * sq.hstride + sq.q_row0;  // row of position 0 of this head
    const int64_t wsrow0 = hh * sq.ws_hstride + sq.ws_row0;
    const uint16_t* kbase = a.k + ((int64_t)g * sq.hstride + sq.kv_row0) * kHeadDim;
    const uint16_t* vbase = a.v + ((int64_t)g * sq.hstride + sq.kv_row0) * kHeadDim;
    const int t_last = pb;
    const int rb = row_base(lane), tb = tr_base(lane);
    DqPlan plan;
#pragma unroll
    for (int k = 0; k < kDqLoadsMax; ++k) {
        const int i = w + kDqWaves * k;
        const int ti = i < kDqTileLoads ? i : i - kDqTileLoads;
        plan.off[k] = i < kDqStageLoads ? perm_src<64>(ti, lane, 63) : 0u;
    }

    dq_stage(kbase, vbase, 0, S, plan, smem, w);
    if (t_last >= 1) dq_stage(kbase, vbase, kTile, S, plan, smem + kDqStageBytes, w);

    // B operands of this wave's rows: Q and dO, lane (row j, half h) holds d = 16 st + 8h .. + 7
    bf16x8 qf[8], df[8];
    float lse2 = 0.0f, Di = 0.0f;
    {
        const int64_t r = active ? pos : S - 1;
        const int64_t qrow = (qrow0 + r) * kHeadDim;
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const u32x4 x4 = *reinterpret_cast<const u32x4*>(a.q + qrow + 16 * st + 8 * h);
            const u32x4 y4 = *reinterpret_cast<const u32x4*>(a.dout + qrow + 16 * st + 8 * h);
            qf[st] = __builtin_bit_cast(bf16x8, active ? x4 : zero);
            df[st] = __builtin_bit_cast(bf16x8, active ? y4 : zero);
        }
        if (active) {
            lse2 = a.ws_lse2[wsrow0 + pos];
            Di = a.ws_d[wsrow0 + pos];
        }
    }
    // complete before the tile loop (see dkdv_body)
    wait_vm<0>();

    f32x16 acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] = zero16();
    const float c = a.c;
    const int grp = w >> 2;
    const int T = t_last;

    // Ping-pong, as in the forward prefill: waves w and w + 4 share a SIMD;
    // group 0 runs tile t as products (dQ of tile t - 1, then S and dP of
    // tile t) followed by the vector work of tile t (P, dS), group 1 the same
    // one step behind.  One barrier per tile, before the products of tile t,
    // after every wave has waited for its own loads of t; the loads of tile
    // t + 2 are issued at the start of the vector work of tile t, into the
    // stage of tile t - 2 (last read, as K^T, in the products of t - 1).
    auto tile_start = [&](int t) {
        if (t <= T) {
            if (t + 1 <= T && grp == 0) {
                if (w < kDqStageLoads - (kDqLoadsMax - 1) * kDqWaves)
                    wait_vm<kDqLoadsMax>();
                else
                    wait_vm<kDqLoadsMax - 1>();
            } else {
                wait_vm<0>();
            }
        }
        __syncthreads();
    };
    f32x16 s[2], dp[2];
    bf16x8 sb[4];
    auto products = [&](int t) {
        __builtin_amdgcn_s_setprio(3);
        if (t >= 1) {
            // dQ^T += K^T dS^T of tile t - 1, the transposed K fragments read two steps ahead
            const char* sK = smem + ((t - 1) % kDqStages) * kDqStageBytes;
            bf16x8 ft[3];
            ft[0] = tr_frag(sK, tb, 0, 0, 0);
            ft[1] = tr_frag(sK, tb, 0, 0, 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                const int ku = x >> 2, db = x & 3;  // ku = 2 kb + u
                if (x + 2 < 16) ft[(x + 2) % 3] = tr_frag(sK, tb, (x + 2) >> 3, ((x + 2) >> 2) & 1, (x + 2) & 3);
                acc[db] = mfma(ft[x % 3], sb[ku], acc[db]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (t <= T) {
            // the 32 products of S^T and dP^T of tile t, each pair's K and V
            // fragments read two steps ahead (scheduling fences keep this order)
            const char* sK = smem + (t % kDqStages) * kDqStageBytes;
            const char* sV = sK + kDqTileBytes;
            s[0] = zero16();
            dp[0] = zero16();
            s[1] = zero16();
            dp[1] = zero16();
            bf16x8 fk[3], fv[3];
            fk[0] = row_frag(sK, rb, 0, 0);
            fv[0] = row_frag(sV, rb, 0, 0);
            fk[1] = row_frag(sK, rb, 0, 1);
            fv[1] = row_frag(sV, rb, 0, 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                const int kb = x >> 3, st = x & 7;
                if (x + 2 < 16) fk[(x + 2) % 3] = row_frag(sK, rb, (x + 2) >> 3, (x + 2) & 7);
                s[kb] = mfma(fk[x % 3], qf[st], s[kb]);
                if (x + 2 < 16) fv[(x + 2) % 3] = row_frag(sV, rb, (x + 2) >> 3, (x + 2) & 7);
                dp[kb] = mfma(fv[x % 3], df[st], dp[kb]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    // P and dS of tile t (bf16 in sb), after issuing this wave's loads of tile t + 2
    auto vector_work = [&](int t) {
        __builtin_amdgcn_s_setprio(0);
        if (t + 2 <= T) dq_stage(kbase, vbase, (int64_t)(t + 2) * kTile, S, plan,
                                 smem + ((t + 2) % kDqStages) * kDqStageBytes, w);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) s[kb][v] = exp2_hw(__builtin_fmaf(s[kb][v], c, -lse2));
        }
        // diagonal tile only (a uniform branch around the selects): element v
        // of block kb is key key0 + 32 kb + 8 (v >> 2) + 4h + (v & 3), visible
        // when that is <= pos, i.e. 32 kb + 8 (v >> 2) + (v & 3) <= vis
        if (t == T) {
            const int vis = (int)(pos - (int64_t)t * kTile) - 4 * h;  // pos - key0 in [0, 63]
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int v = 0; v < 16; ++v) s[kb][v] = 32 * kb + 8 * (v >> 2) + (v & 3) <= vis ? s[kb][v] : 0.0f;
            }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) dp[kb][v] = s[kb][v] * (dp[kb][v] - Di);
        }
        sb[0] = pack8(dp[0], 0);
        sb[1] = pack8(dp[0], 1);
        sb[2] = pack8(dp[1], 0);
        sb[3] = pack8(dp[1], 1);
    };
    if (grp == 0) {
        for (int t = 0; t <= T; ++t) {
            tile_start(t);
            products(t);
            vector_work(t);
        }
        tile_start(T + 1);
        products(T + 1);
    } else {
        tile_start(0);
        products(0);
        for (int t = 0; t <= T; ++t) {
            tile_start(t + 1);
            vector_work(t);
            products(t + 1);
        }
    }
    __builtin_amdgcn_s_setprio(0);

    if (active) store_col(a.dq + (qrow0 + pos) * kHeadDim, acc, a.scale, h);
}

// Dense batch: [B, H, S, 128].
__global__ __launch_bounds__(64 * kDqWaves) void bwd_dq_kernel(BwdArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[kDqStages * kDqStageBytes];
    const int n_pb = (int)((a.seq_len + 63) / 64);
    const int nbg = a.batch * a.n_kv_heads;
    const int x = blockIdx.x;
    int bg, pbr;
    if ((nbg & 7) == 0) {
        const int i = x >> 3;
        bg = (i / n_pb) * 8 + (x & 7);
        pbr = i % n_pb;
    } else {
        bg = x % nbg;
        pbr = x / nbg;
    }
    // longest rows first
    dq_body(a, dense_seq(a, bg / a.n_kv_heads), bg % a.n_kv_heads, n_pb - 1 - pbr, smem);
}

// Ragged batch (packed [H, T, 128]): units of a sequence are (64-row block,
// KV head), longest blocks first.
__global__ __launch_bounds__(64 * kDqWaves) void bwd_dq_varlen_kernel(BwdArgs a, BwdTable t) {
    __shared__ __attribute__((aligned(1024))) char smem[kDqStages * kDqStageBytes];
    const int x = blockIdx.x;
    int s = 0;
    while (s + 1 < t.n_seqs && t.unit_dq[s + 1] <= x) ++s;
    const int u = x - t.unit_dq[s];
    const int n_pb = (t.len[s] + 63) / 64;
    dq_body(a, table_seq(t, s), u % a.n_kv_heads, n_pb - 1 - u / a.n_kv_heads, smem);
}

}  // namespace bwd
}  // namespace kb

using namespace kb;
using namespace kb::bwd;

namespace {

constexpr int64_t kMaxSeq = int64_t(1) << 30;

bool overlap(const void* a, size_t an, const void* b, size_t bn) {
    if (!a || !b || !an || !bn) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

int on_device(std::initializer_list<const void*> ptrs) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return KB_ATTN_ERR_DEVICE;
    }
    for (const void* p : ptrs) {
        hipPointerAttribute_t attr;
        if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
            (void)hipGetLastError();
            return KB_ATTN_ERR_DEVICE;
        }
        if (attr.type != hipMemoryTypeDevice || attr.device != dev) return KB_ATTN_ERR_DEVICE;
    }
    return KB_ATTN_OK;
}

int64_t padded_rows(int64_t seq_len) { return (seq_len + 63) / 64 * 64; }

// Checks a ragged batch's host offsets (batch + 1 entries, from >= 0,
// non-decreasing, each sequence at most kMaxSeq rows) and returns the packed
// row count and the padded workspace rows (each sequence padded to 64).
int ragged_rows(const int64_t* cu, int64_t batch, int64_t* t_rows, int64_t* t_pad) {
    if (cu[0] < 0) return KB_ATTN_ERR_LENGTH;
    int64_t pad = 0;
    for (int64_t i = 0; i < batch; ++i) {
        const int64_t len = cu[i + 1] - cu[i];
        if (len < 0 || len > kMaxSeq) return KB_ATTN_ERR_LENGTH;
        pad += padded_rows(len);
    }
    if (cu[batch] > (kMaxSeq << 6) || pad > (kMaxSeq << 6)) return KB_ATTN_ERR_LENGTH;
    if (t_rows) *t_rows = cu[batch];
    if (t_pad) *t_pad = pad;
    return KB_ATTN_OK;
}

}  // namespace

extern "C" {

size_t kb_attn_backward_workspace_bytes(int64_t batch, int64_t seq_len, int32_t n_q_heads, int32_t head_dim) {
    if (batch < 1 || seq_len < 1 || seq_len > kMaxSeq || n_q_heads < 1 || head_dim != kHeadDim) return 0;
    return (size_t)2 * batch * n_q_heads * padded_rows(seq_len) * sizeof(float);
}

int kb_attn_backward(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                     void* dq, void* dk, void* dv, int64_t batch, int64_t seq_len, int32_t n_q_heads,
                     int32_t n_kv_heads, int32_t head_dim, float scale, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || batch < 1 || seq_len < 1)
        return KB_ATTN_ERR_INVALID_ARG;
    if (n_q_heads < 1 || n_kv_heads < 1 || head_dim < 1) return KB_ATTN_ERR_INVALID_ARG;
    if (head_dim != kHeadDim || n_q_heads != kGroup * n_kv_heads) return KB_ATTN_ERR_UNSUPPORTED;
    if (!(scale > 0.0f) || !(scale < __builtin_inff())) return KB_ATTN_ERR_INVALID_ARG;
    if (seq_len > kMaxSeq || batch * n_kv_heads > INT32_MAX) return KB_ATTN_ERR_LENGTH;
    const size_t need = kb_attn_backward_workspace_bytes(batch, seq_len, n_q_heads, head_dim);
    if (!workspace || workspace_bytes < need) return KB_ATTN_ERR_WORKSPACE;
    for (const void* p : {q, k, v, o, dout, (const void*)dq, (const void*)dk, (const void*)dv, (const void*)workspace})
        if ((uintptr_t)p & 15u) return KB_ATTN_ERR_ALIGNMENT;
    if ((uintptr_t)lse & 3u) return KB_ATTN_ERR_ALIGNMENT;

    const size_t qb = (size_t)batch * n_q_heads * seq_len * kHeadDim * 2;
    const size_t kb_ = (size_t)batch * n_kv_heads * seq_len * kHeadDim * 2;
    const size_t lb = (size_t)batch * n_q_heads * seq_len * sizeof(float);
    const std::pair<const void*, size_t> outs[] = {{dq, qb}, {dk, kb_}, {dv, kb_}, {workspace, need}};
    const std::pair<const void*, size_t> ins[] = {{q, qb}, {k, kb_}, {v, kb_}, {o, qb}, {dout, qb}, {lse, lb}};
    for (size_t i = 0; i < 4; ++i) {
        for (size_t m = i + 1; m < 4; ++m)
            if (overlap(outs[i].first, outs[i].second, outs[m].first, outs[m].second)) return KB_ATTN_ERR_ALIAS;
        for (const auto& in : ins)
            if (overlap(outs[i].first, outs[i].second, in.first, in.second)) return KB_ATTN_ERR_ALIAS;
    }
    if (int rc = on_device({q, k, v, o, dout, lse, dq, dk, dv, workspace})) return rc;

    BwdArgs a;
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.o = (const uint16_t*)o;
    a.dout = (const uint16_t*)dout;
    a.lse = lse;
    a.dq = (uint16_t*)dq;
    a.dk = (uint16_t*)dk;
    a.dv = (uint16_t*)dv;
    a.seq_len = seq_len;
    a.s_pad = padded_rows(seq_len);
    a.ws_d = (float*)workspace;
    a.ws_lse2 = (float*)workspace + (int64_t)batch * n_q_heads * a.s_pad;
    a.batch = (int32_t)batch;
    a.n_kv_heads = n_kv_heads;
    a.c = (float)((double)scale * 1.4426950408889634073599246810019);
    a.scale = scale;

    const int64_t prep_rows = (int64_t)batch * n_q_heads * a.s_pad;
    const int64_t prep_grid = (prep_rows + 31) / 32;
    const int64_t nbg = batch * n_kv_heads;
    const int64_t kv_grid = nbg * ((seq_len + kKvKeys - 1) / kKvKeys);
    const int64_t dq_grid = nbg * ((seq_len + 63) / 64);
    if (prep_grid > INT32_MAX || kv_grid > INT32_MAX || dq_grid > INT32_MAX) return KB_ATTN_ERR_LENGTH;
    hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)prep_grid), dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return KB_ATTN_ERR_HIP;
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)kv_grid), dim3(64 * kKvWaves), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return KB_ATTN_ERR_HIP;
    hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)dq_grid), dim3(64 * kDqWaves), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return KB_ATTN_ERR_HIP;
    return KB_ATTN_OK;
}

size_t kb_attn_backward_varlen_workspace_bytes(const int64_t* cu_seqlens, int64_t batch, int32_t n_q_heads,
                                               int32_t head_dim) {
    if (!cu_seqlens || batch < 1 || n_q_heads < 1 || head_dim != kHeadDim) return 0;
    int64_t t_pad = 0;
    if (ragged_rows(cu_seqlens, batch, nullptr, &t_pad) != KB_ATTN_OK) return 0;
    return (size_t)2 * n_q_heads * t_pad * sizeof(float);
}

int kb_attn_backward_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, void* dq, void* dk, void* dv, const int64_t* cu_seqlens, int64_t batch,
                            int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float scale, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !cu_seqlens || batch < 1)
        return KB_ATTN_ERR_INVALID_ARG;
    if (n_q_heads < 1 || n_kv_heads < 1 || head_dim < 1) return KB_ATTN_ERR_INVALID_ARG;
    if (head_dim != kHeadDim || n_q_heads != kGroup * n_kv_heads) return KB_ATTN_ERR_UNSUPPORTED;
    if (!(scale > 0.0f) || !(scale < __builtin_inff())) return KB_ATTN_ERR_INVALID_ARG;
    int64_t t_rows = 0, t_pad = 0;
    if (int rc = ragged_rows(cu_seqlens, batch, &t_rows, &t_pad)) return rc;
    const size_t need = (size_t)2 * n_q_heads * t_pad * sizeof(float);
    if (need && (!workspace || workspace_bytes < need)) return KB_ATTN_ERR_WORKSPACE;
    for (const void* p : {q, k, v, o, dout, (const void*)dq, (const void*)dk, (const void*)dv})
        if ((uintptr_t)p & 15u) return KB_ATTN_ERR_ALIGNMENT;
    if (need && ((uintptr_t)workspace & 15u)) return KB_ATTN_ERR_ALIGNMENT;
    if ((uintptr_t)lse & 3u) return KB_ATTN_ERR_ALIGNMENT;
    const size_t qb = (size_t)n_q_heads * t_rows * kHeadDim * 2;
    const size_t kb_ = (size_t)n_kv_heads * t_rows * kHeadDim * 2;
    const size_t lb = (size_t)n_q_heads * t_rows * sizeof(float);
    const std::pair<const void*, size_t> outs[] = {{dq, qb}, {dk, kb_}, {dv, kb_}, {need ? workspace : nullptr, need}};
    const std::pair<const void*, size_t> ins[] = {{q, qb}, {k, kb_}, {v, kb_}, {o, qb}, {dout, qb}, {lse, lb}};
    for (size_t i = 0; i < 4; ++i) {
        for (size_t m = i + 1; m < 4; ++m)
            if (overlap(outs[i].first, outs[i].second, outs[m].first, outs[m].second)) return KB_ATTN_ERR_ALIAS;
        for (const auto& in : ins)
            if (overlap(outs[i].first, outs[i].second, in.first, in.second)) return KB_ATTN_ERR_ALIAS;
    }
    if (int rc = on_device({q, k, v, o, dout, lse, dq, dk, dv})) return rc;
    if (need)
        if (int rc = on_device({workspace})) return rc;
    if (t_rows == 0) return KB_ATTN_OK;  // every sequence is empty

    BwdArgs a;
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.o = (const uint16_t*)o;
    a.dout = (const uint16_t*)dout;
    a.lse = lse;
    a.dq = (uint16_t*)dq;
    a.dk = (uint16_t*)dk;
    a.dv = (uint16_t*)dv;
    a.seq_len = 0;  // per sequence, from the table
    a.s_pad = 0;
    a.ws_d = (float*)workspace;
    a.ws_lse2 = (float*)workspace + (int64_t)n_q_heads * t_pad;
    a.batch = 0;
    a.n_kv_heads = n_kv_heads;
    a.c = (float)((double)scale * 1.4426950408889634073599246810019);
    a.scale = scale;

    // sequences in the caller's order, at most kBwdMaxSeqs non-empty ones per
    // launch (a sequence's bits do not depend on which launch carries it)
    int64_t pad = 0;
    int64_t i = 0;
    while (i < batch) {
        BwdTable t;
        t.n_seqs = 0;
        t.t_rows = t_rows;
        t.t_pad = t_pad;
        t.p_begin = pad;
        int64_t units_kv = 0, units_dq = 0;
        for (; i < batch && t.n_seqs < kBwdMaxSeqs; ++i) {
            const int64_t len = cu_seqlens[i + 1] - cu_seqlens[i];
            if (len == 0) continue;
            const int n = t.n_seqs++;
            t.row0[n] = cu_seqlens[i];
            t.pad0[n] = pad;
            t.len[n] = (int32_t)len;
            t.unit_kv[n] = (int32_t)units_kv;
            t.unit_dq[n] = (int32_t)units_dq;
            units_kv += (int64_t)n_kv_heads * ((len + kKvKeys - 1) / kKvKeys);
            units_dq += (int64_t)n_kv_heads * ((len + 63) / 64);
            pad += padded_rows(len);
            if (units_kv > INT32_MAX || units_dq > INT32_MAX) return KB_ATTN_ERR_LENGTH;
        }
        if (t.n_seqs == 0) break;
        t.unit_kv[t.n_seqs] = (int32_t)units_kv;
        t.unit_dq[t.n_seqs] = (int32_t)units_dq;
        t.p_count = pad - t.p_begin;
        const int64_t prep_grid = (int64_t)n_q_heads * (t.p_count / 32);
        if (prep_grid > INT32_MAX) return KB_ATTN_ERR_LENGTH;
        hipLaunchKernelGGL(bwd_prep_varlen_kernel, dim3((unsigned)prep_grid), dim3(256), 0, stream, a, t);
        if (hipGetLastError() != hipSuccess) return KB_ATTN_ERR_HIP;
        hipLaunchKernelGGL(bwd_dkdv_varlen_kernel, dim3((unsigned)units_kv), dim3(64 * kKvWaves), 0, stream, a, t);
        if (hipGetLastError() != hipSuccess) return KB_ATTN_ERR_HIP;
        hipLaunchKernelGGL(bwd_dq_varlen_kernel, dim3((unsigned)units_dq), dim3(64 * kDqWaves), 0, stream, a, t);
        if (hipGetLastError() != hipSuccess) return KB_ATTN_ERR_HIP;
    }
    return KB_ATTN_OK;
}

}  // extern "C"
