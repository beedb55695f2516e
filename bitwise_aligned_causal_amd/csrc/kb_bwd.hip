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
//   bwd_dkdv_kernel  two waves per 32 keys of a KV head (192 keys, 12 waves
//                    per workgroup); the Q / dO rows of
//                    the 4 query heads stream through LDS in 32-row tiles:
//                      S    = Q K^T           (A = Q rows,  B = K rows in registers)
//                      P    = exp2(S c - lse2),  dV^T += dO^T P        (first wave)
//                      dP   = dO V^T          (A = dO rows, B = V rows in registers)
//                      dS   = P (dP - D),  dK^T += Q^T dS            (second wave)
//                    (the second operands read transposed from LDS; P passes
//                    from the first wave to the second through LDS)
//   bwd_dq_kernel    one wave per 32 query rows; K / V tiles of 64 keys stream
//                    through LDS as in the forward:
//                      S^T  = K Q^T,  dP^T = V dO^T,  dQ^T += K^T dS^T
// All products are v_mfma_f32_32x32x16_bf16 with fp32 accumulation; P and dS
// are rounded to bf16 (RNE) as the operands of the second products.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <initializer_list>

#include "../../include/kb_attn.h"
#include "kb_contract.h"

namespace kb {
namespace bwd {

// ---------------------------------------------------------------------------
// LDS tiles: rows of 256 bytes (128 bf16), 16-byte chunk c of row r stored at
// chunk position c ^ swz(r).  Tiles read both by rows and transposed use
//   dual(r) = ((r & 3) << 2) | ((r >> 2) & 3)
// which gives 16 distinct positions for the row reads (16 consecutive rows,
// one chunk) and for the transposing reads (4 consecutive rows x 4
// consecutive chunks); tiles read only by rows use r & 15.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int dual_swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

template <bool kDual>
__device__ __forceinline__ int swz(int row) {
    return kDual ? dual_swz(row) : (row & 15);
}

// Direct-to-LDS loads of a tile of 64 rows row0 .. row0 + 63 of a [rows, 128]
// bf16 matrix; rows beyond last_row read last_row (they are masked or
// weighted by zero later).  Instruction i (0..15) fills tile rows 4i .. 4i + 3,
// lane L landing at tile byte 1024 i + 16 L; the wave issues instructions
// first, first + step, ... (a rolled loop: it keeps no per-instruction
// addresses live across the caller's loop).
template <bool kDual>
__device__ __forceinline__ void stage_rows(const uint16_t* base, int64_t row0, int64_t last_row, char* tile,
                                           int first, int step, int lane) {
    const char* tb = reinterpret_cast<const char*>(base + row0 * kHeadDim);
    const int64_t last = last_row - row0;
    for (int i = first; i < 16; i += step) {
        const int row = 4 * i + (lane >> 4);
        const int c = (lane & 15) ^ swz<kDual>(row);
        const int64_t r = row < last ? row : last;
        lds_dma16(tb, (uint32_t)(r * 256 + c * 16), tile + 1024 * i);
    }
}

// lds_dma16 with the scalar base forced into scalar registers: the base is
// uniform by construction, but the compiler cannot always prove it.
__device__ __forceinline__ void dma16(const char* base, uint32_t voff, char* dst) {
    const uint64_t p = (uint64_t)(uintptr_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    lds_dma16(reinterpret_cast<const char*>((uintptr_t)(((uint64_t)hi << 32) | lo)), voff, dst);
}

// Row fragment: lane (row 32 blk + (lane & 31), half h) holds bf16
// [16 st + 8h, 16 st + 8h + 7] of its row -- the A operand of a product whose
// rows are the tile's rows, or the B operand whose columns are.
template <bool kDual>
__device__ __forceinline__ bf16x8 row_frag(const char* tile, int blk, int st, int lane) {
    const int row = 32 * blk + (lane & 31);
    const int c = 2 * st + (lane >> 5);
    return lds_read16(tile + row * 256 + ((c ^ swz<kDual>(row)) << 4));
}

// Transposed fragment (dual swizzle): the A operand X^T[d][rows] for d block
// dblk and the 16-row step (blk, u) of the tile, with the row order of an
// MFMA result column: lane (d = 32 dblk + j, half h) holds, in slot order,
//   X[R0 + 4h + {0..3}][d], X[R0 + 8 + 4h + {0..3}][d],   R0 = 32 blk + 16 u
// (two ds_read_b64_tr_b16; same addressing as the forward's V^T reads).
__device__ __forceinline__ bf16x8 tr_frag(const char* tile, int blk, int u, int dblk, int lane) {
    const int g = lane >> 4, n = (lane >> 2) & 3, jj = lane & 3;
    const int row0 = 32 * blk + 16 * u + 4 * (g >> 1) + n;
    const int d = 32 * dblk + 16 * (g & 1) + 4 * jj;
    const int c = d >> 3, half = (d & 4) << 1;
    const int row1 = row0 + 8;
    const char* p0 = tile + row0 * 256 + ((c ^ dual_swz(row0)) << 4) + half;
    const char* p1 = tile + row1 * 256 + ((c ^ dual_swz(row1)) << 4) + half;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
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
// dK/dV and dQ work units (KV heads x 192-key blocks, KV heads x 64-row
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
// dK, dV: workgroup = 12 waves on 192 keys [K0, K0 + 192) of one (sequence,
// KV head).  Key group kg = w % 6 covers keys k0 = K0 + 32 kg .. + 31 and is
// served by two waves:
//   P-wave  (w < 6)   S = Q K^T, P = exp2(S c - lse2), P to LDS, dV^T += dO^T P
//   dS-wave (w >= 6)  one item later: dP = dO V^T, P from LDS,
//                     dS = P (dP - D), dK^T += Q^T dS
// so each wave holds one accumulator set (64 registers) and one of K, V, and
// fits in the 168 registers that let three waves share a SIMD.
// Work items t = 0, 1, ...: query tile q0 = qlast - 32 (t / 4) of query head
// 4g + (t % 4), from the last tile qlast down to K0.  A 4-stage LDS ring holds
// each item's Q rows, dO rows (dual swizzle) and its 32 lse2 and 32 D values,
// loaded two items ahead; P goes through a double buffer.  dK^T and dV^T
// accumulate over the items in that fixed order.
// ---------------------------------------------------------------------------
constexpr int kKvWaves = 12;
constexpr int kKvGroups = 6;
constexpr int kKvKeys = 32 * kKvGroups;
constexpr int kQTileBytes = 32 * 256;
constexpr int kKvStageBytes = 2 * kQTileBytes + 256;  // Q, dO, lse2[32], D[32]
constexpr int kKvStages = 4;
constexpr int kPBufBytes = kKvGroups * 4096;          // fp32 P of the key groups
constexpr int kKvLoadsPerWave = 3;  // waves 0..7: 2 tile loads + 1 block of 8 floats; waves 8..11: none

__device__ __forceinline__ void kv_stage(const BwdArgs& a, const BwdSeq& sq, int g, int t, int64_t qlast,
                                         char* stage, int w, int lane) {
    const int64_t q0 = qlast - 32 * (t >> 2);
    const int64_t hh = kGroup * g + (t & 3);  // query head of the item
    const int64_t qrow = hh * sq.hstride + sq.q_row0 + q0;
    const char* qb = reinterpret_cast<const char*>(a.q + qrow * kHeadDim);
    const char* db = reinterpret_cast<const char*>(a.dout + qrow * kHeadDim);
    const int64_t last = sq.S - 1 - q0;  // last valid row, relative to q0
    // waves 0..7 issue the stage's loads (waves 8..11 none): instructions 0..7
    // fill Q rows 4i..4i+3, 8..15 fill dO; wave w issues w and w + 8
    if (w >= 8) return;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int i = w + 8 * k;
        const int row = 4 * (i & 7) + (lane >> 4);
        const int c = (lane & 15) ^ dual_swz(row);
        const int64_t r = row < last ? row : last;
        dma16(i < 8 ? qb : db, (uint32_t)(r * 256 + c * 16), stage + 1024 * i);
    }
    // lse2 / D of the 32 rows (padded arrays, in bounds): wave w moves 8
    // floats with lanes 0..1 (w < 4: lse2[8w ..], else D[8(w-4) ..])
    const float* src = (w < 4 ? a.ws_lse2 : a.ws_d) + hh * sq.ws_hstride + sq.ws_row0 + q0 + 8 * (w & 3);
    if (lane < 2) dma16(reinterpret_cast<const char*>(src), (uint32_t)(lane * 16), stage + 2 * kQTileBytes + 32 * w);
}

// Everything a dK/dV wave needs once its work item is known.
struct KvWork {
    BwdSeq sq;
    int g;
    int64_t S, K0, k0, qlast;
    int n_items, kg, w, lane;
    char* smem;
    char* pbuf;
};

// P-wave part of one item: S = Q K^T, P (masked on edge tiles), P to LDS,
// dV^T += dO^T P.  Element v: query q0 + 8 (v >> 2) + 4h + (v & 3), key
// k0 + j; on an edge tile it counts when k0 + j <= query < S, i.e.
// lo <= 8 (v >> 2) + (v & 3) < hi.  The mask is a uniform branch around the
// selects only, so the accumulators never cross a join.
__device__ __forceinline__ void p_item(const bf16x8 (&kf)[8], const char* sQ, const char* sD, const float* sL,
                                       float4* pb4, int lane, float c, bool edge, int lo, int hi,
                                       f32x16 (&acc)[4]) {
    const int h = lane >> 5;
    f32x16 s = zero16();
#pragma unroll
    for (int st = 0; st < 8; ++st) s = mfma(row_frag<true>(sQ, 0, st, lane), kf[st], s);
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
    for (int b4 = 0; b4 < 4; ++b4)
        pb4[b4 * 64 + lane] = make_float4(s[4 * b4], s[4 * b4 + 1], s[4 * b4 + 2], s[4 * b4 + 3]);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const bf16x8 pb = pack8(s, u);
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[db] = mfma(tr_frag(sD, 0, u, db, lane), pb, acc[db]);
    }
}

// dS-wave part of one item: dP = dO V^T, P from LDS, dS = P (dP - D),
// dK^T += Q^T dS.
__device__ __forceinline__ void ds_item(const bf16x8 (&vf)[8], const char* sQ, const char* sD, const float* sL,
                                        const float4* pb4, int lane, f32x16 (&acc)[4]) {
    const int h = lane >> 5;
    f32x16 dp = zero16();
#pragma unroll
    for (int st = 0; st < 8; ++st) dp = mfma(row_frag<true>(sD, 0, st, lane), vf[st], dp);
#pragma unroll
    for (int b4 = 0; b4 < 4; ++b4) {
        const float4 p4 = pb4[b4 * 64 + lane];
        const float4 d4 = *reinterpret_cast<const float4*>(sL + 32 + 8 * b4 + 4 * h);
        const float pv[4] = {p4.x, p4.y, p4.z, p4.w};
        const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) dp[4 * b4 + i] = pv[i] * (dp[4 * b4 + i] - dv[i]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const bf16x8 sb = pack8(dp, u);
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[db] = mfma(tr_frag(sQ, 0, u, db, lane), sb, acc[db]);
    }
}

// The item loop of one role (both roles run the same iterations and
// barriers; the P-wave works on item t, the dS-wave on item t - 1).  Each
// role has its own loop so that its accumulators stay in place.
template <bool kP>
__device__ __forceinline__ void kv_loop(const BwdArgs& a, const KvWork& wk, const bf16x8 (&kvf)[8],
                                        f32x16 (&acc)[4]) {
    const int lane = wk.lane, j = lane & 31, h = lane >> 5;
    const float c = a.c;
    for (int t = 0; t <= wk.n_items; ++t) {
        // publish item t's stage (the item t + 1 stage may still be loading), refill
        if (t + 1 < wk.n_items)
            wait_vm<kKvLoadsPerWave>();
        else
            wait_vm<0>();
        __syncthreads();
        if (t + 2 < wk.n_items)
            kv_stage(a, wk.sq, wk.g, t + 2, wk.qlast, wk.smem + ((t + 2) % kKvStages) * kKvStageBytes, wk.w, lane);

        const int it = kP ? t : t - 1;
        if (it < 0 || it >= wk.n_items) continue;
        const int64_t q0 = wk.qlast - 32 * (it >> 2);
        if (q0 < wk.k0) continue;  // every key of this group lies after every row of the tile
        const char* stage = wk.smem + (it % kKvStages) * kKvStageBytes;
        const char* sQ = stage;
        const char* sD = stage + kQTileBytes;
        const float* sL = reinterpret_cast<const float*>(stage + 2 * kQTileBytes);
        float4* pb4 = reinterpret_cast<float4*>(wk.pbuf + (it & 1) * kPBufBytes + wk.kg * 4096);
        if (kP) {
            const bool edge = q0 == wk.k0 || q0 + 32 > wk.S;
            const int lo = (int)(wk.k0 - q0) + j - 4 * h;
            const int hi = (int)(wk.S - q0 < 64 ? wk.S - q0 : 64) - 4 * h;
            p_item(kvf, sQ, sD, sL, pb4, lane, c, edge, lo, hi, acc);
        } else {
            ds_item(kvf, sQ, sD, sL, pb4, lane, acc);
        }
    }
}

// One dK/dV workgroup: keys [192 kb, 192 kb + 192) of KV head g of one sequence.
__device__ __forceinline__ void dkdv_body(const BwdArgs& a, const BwdSeq& sq, int g, int kb, char* smem) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = w % kKvGroups;
    const bool pwave = w < kKvGroups;
    const int j = lane & 31, h = lane >> 5;
    KvWork wk;
    wk.sq = sq;
    wk.g = g;
    wk.S = sq.S;
    wk.K0 = (int64_t)kb * kKvKeys;
    wk.k0 = wk.K0 + 32 * kg;  // this wave's first key
    // query tiles from the last one down to K0: every block of a (sequence,
    // KV head) starts at the same rows, so the blocks running together on an
    // XCD read the same Q / dO rows at about the same time (one L2 fetch)
    wk.qlast = ((wk.S - 1) >> 5) << 5;
    wk.n_items = 4 * (int)((wk.qlast - wk.K0) / 32 + 1);
    wk.kg = kg;
    wk.w = w;
    wk.lane = lane;
    wk.smem = smem;
    wk.pbuf = smem + kKvStages * kKvStageBytes;
    const int64_t S = wk.S;

    kv_stage(a, sq, g, 0, wk.qlast, smem, w, lane);
    if (wk.n_items >= 2) kv_stage(a, sq, g, 1, wk.qlast, smem + kKvStageBytes, w, lane);

    // this wave's K (P-wave) or V (dS-wave) rows as B operands: lane (key j,
    // half h) holds row k0 + j, d = 16 st + 8h .. + 7 (rows beyond S read row S - 1)
    const int64_t kv0 = (int64_t)g * sq.hstride + sq.kv_row0;  // row of key 0
    bf16x8 kvf[8];
    {
        int64_t key = wk.k0 + j;
        key = key < S ? key : S - 1;
        const uint16_t* src = (pwave ? a.k : a.v) + (kv0 + key) * kHeadDim;
#pragma unroll
        for (int st = 0; st < 8; ++st)
            kvf[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src + 16 * st + 8 * h));
    }

    f32x16 acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] = zero16();
    const int64_t row = (kv0 + wk.k0 + j) * kHeadDim;
    if (pwave) {
        kv_loop<true>(a, wk, kvf, acc);
        if (wk.k0 + j < S) store_col(a.dv + row, acc, 1.0f, h);
    } else {
        kv_loop<false>(a, wk, kvf, acc);
        if (wk.k0 + j < S) store_col(a.dk + row, acc, a.scale, h);
    }
}

// Dense batch: [B, H, S, 128].
__global__ __launch_bounds__(64 * kKvWaves) void bwd_dkdv_kernel(BwdArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[kKvStages * kKvStageBytes + 2 * kPBufBytes];
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

// Ragged batch (packed [H, T, 128]): units of a sequence are (192-key block,
// KV head), longest blocks first.
__global__ __launch_bounds__(64 * kKvWaves) void bwd_dkdv_varlen_kernel(BwdArgs a, BwdTable t) {
    __shared__ __attribute__((aligned(1024))) char smem[kKvStages * kKvStageBytes + 2 * kPBufBytes];
    const int x = blockIdx.x;
    int s = 0;
    while (s + 1 < t.n_seqs && t.unit_kv[s + 1] <= x) ++s;
    const int u = x - t.unit_kv[s];
    dkdv_body(a, table_seq(t, s), u % a.n_kv_heads, u / a.n_kv_heads, smem);
}

// ---------------------------------------------------------------------------
// dQ: workgroup = 8 waves = the 4 query heads of one KV head x 2 halves of
// the 64 positions [64 pb, 64 pb + 64), as in the forward; K / V tiles of 64
// keys (K dual-swizzled, V rows only) stream through a 3-stage ring, loads two
// tiles ahead.  Wave column j is query row 64 pb + 32 (w >> 2) + j.
// ---------------------------------------------------------------------------
constexpr int kDqWaves = 8;
constexpr int kDqStages = 3;
constexpr int kDqLoadsPerWave = kTileLoads / kDqWaves;

__device__ __forceinline__ void dq_stage(const uint16_t* kb, const uint16_t* vb, int64_t key0, int64_t last,
                                         char* stage, int w, int lane) {
    stage_rows<true>(kb, key0, last, stage, w, kDqWaves, lane);
    stage_rows<false>(vb, key0, last, stage + kKBytes, w, kDqWaves, lane);
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

    dq_stage(kbase, vbase, 0, S - 1, smem, w, lane);
    if (t_last >= 1) dq_stage(kbase, vbase, kTile, S - 1, smem + kTileBytes, w, lane);

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

    f32x16 acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] = zero16();
    const float c = a.c;

    for (int t = 0; t <= t_last; ++t) {
        if (t + 1 <= t_last)
            wait_vm<kDqLoadsPerWave>();
        else
            wait_vm<0>();
        __syncthreads();
        if (t + 2 <= t_last) {
            char* nb = smem + ((t + 2) % kDqStages) * kTileBytes;
            dq_stage(kbase, vbase, (int64_t)(t + 2) * kTile, S - 1, nb, w, lane);
        }
        const char* sK = smem + (t % kDqStages) * kTileBytes;
        const char* sV = sK + kKBytes;
        const int64_t key0 = (int64_t)t * kTile;

        f32x16 s[2], dp[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = zero16();
            dp[kb] = zero16();
#pragma unroll
            for (int st = 0; st < 8; ++st) {
                s[kb] = mfma(row_frag<true>(sK, kb, st, lane), qf[st], s[kb]);
                dp[kb] = mfma(row_frag<false>(sV, kb, st, lane), df[st], dp[kb]);
            }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) s[kb][v] = exp2_hw(__builtin_fmaf(s[kb][v], c, -lse2));
        }
        // diagonal tile only (a uniform branch around the selects): element v
        // of block kb is key key0 + 32 kb + 8 (v >> 2) + 4h + (v & 3), visible
        // when that is <= pos, i.e. 32 kb + 8 (v >> 2) + (v & 3) <= vis
        if (t == t_last) {
            const int vis = (int)(pos - key0) - 4 * h;  // pos - key0 in [0, 63]
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
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const bf16x8 sb = pack8(dp[kb], u);
#pragma unroll
                for (int db = 0; db < 4; ++db) acc[db] = mfma(tr_frag(sK, kb, u, db, lane), sb, acc[db]);
            }
        }
    }

    if (active) store_col(a.dq + (qrow0 + pos) * kHeadDim, acc, a.scale, h);
}

// Dense batch: [B, H, S, 128].
__global__ __launch_bounds__(64 * kDqWaves) void bwd_dq_kernel(BwdArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[kDqStages * kTileBytes];
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
    __shared__ __attribute__((aligned(1024))) char smem[kDqStages * kTileBytes];
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
