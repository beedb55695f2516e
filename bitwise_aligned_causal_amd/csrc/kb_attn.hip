// kb_attn: bitwise-aligned causal GQA attention forward for gfx950 (MI355X).
//
// Three kernels, all built on the contract in kb_contract.h:
//   prefill_kernel  full-sequence prefill and partitioned forward (the same
//                   kernel: row r sits at position kv_len - q_len + r); one
//                   workgroup per 64-position block, or, for launches of 2 to
//                   16 blocks per CU, prefill_persistent_kernel: one
//                   workgroup per CU walking a fixed list of blocks
//   decode_kernel   one query token; the 4 query heads of a KV head share
//                   one MFMA tile (columns 0..3); one workgroup per
//                   (batch, KV head, chunk of 1024 keys)
//   combine_kernel  folds the decode chunks in chunk order
// and the C-ABI of include/kb_attn.h (validation and launch).
//
// Operator: KernelBraid / AReaL-TIK README, "Features" (BF16, causal,
// [batch, heads, seq, head_dim], 32/8 heads, D = 128), "Usage"
// (unified_prefill, unified_decode, output shaped like q, decode equals the
// last prefill row bit for bit) and "Method" (one contract across prefill,
// partitioned forward and decode).
#include <hip/hip_runtime.h>

#include <cmath>
#include <algorithm>
#include <cstdint>
#include <initializer_list>
#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

#include "../../include/kb_attn.h"
#include "kb_contract.h"

namespace kb {

static_assert(KB_ATTN_KV_TILE == kTile && KB_ATTN_KV_CHUNK == kChunk, "header and contract disagree");

struct PrefillArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;  // optional: [batch, Hq, q_len] log-sum-exp of each row
    int64_t q_len, kv_len, cap;
    int32_t batch, n_kv_heads;
    int32_t pb_first, n_pb;  // 64-position blocks covered by the call
    float c;                 // scale * log2(e), rounded once to fp32
};

constexpr int kPrefillWaves = 8;

// Everything a prefill workgroup needs once its work item is known.
struct PrefillWork {
    const uint16_t* q0;  // row 0 of this (sequence, KV head group): query head 4g + i at q0 + i * q_hstride rows
    uint16_t* o0;        // same for the output
    float* lse0;         // optional log-sum-exp output: head 4g + i, row r at lse0[i * q_hstride + r]
    int64_t q_hstride;   // rows between consecutive query heads
    const uint16_t* kbase;  // key 0 of this (sequence, KV head)
    const uint16_t* vbase;
    int64_t q_len, kv_len;
    int pb;  // 64-position block
};

// Workgroup = 8 waves = the 4 query heads of one KV head x 2 halves of the 64
// absolute positions [64 pb, 64 pb + 64).  Every row of the block has its last
// visible key in tile pb, so all rows visit exactly the tiles 0..pb and never
// a tile that is fully masked for them.  K/V tiles are shared by the 8 waves
// through a 4-stage LDS ring (padded rows, PaddedTile) filled by direct loads.
// kPartitioned = false is the full-sequence case (q_len == kv_len, row r at
// position r); both instantiations run the same per-row arithmetic.
//
// Ping-pong: waves w and w + 4 share a SIMD.  Group 0 (waves 0-3) runs tile t
// as products then softmax, group 1 (waves 4-7) one step behind as softmax of
// tile t - 1 then products, so while one wave of a SIMD multiplies the other
// runs its vector work:
//   products(t)  P V of tile t - 1 (pv_fenced), then the scores of tile t
//                (qk_fenced); wave priority 3, so its MFMAs issue first
//   softmax(t)   softmax_tile of tile t at priority 0, after issuing this
//                wave's share of the direct loads of tile t + 2
// One barrier per tile: before the products of tile t every wave has waited
// for its loads of tile t and is past all reads of tile t - 2, whose stage
// tile t + 2 then takes.
constexpr int kStages = 4;

template <bool kPartitioned>
__device__ __forceinline__ void prefill_body(const PrefillWork& wk, float c, char* smem) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = w >> 2;
    const int pb = wk.pb;
    const int j = lane & 31, h = lane >> 5;

    const int64_t off = kPartitioned ? wk.kv_len - wk.q_len : 0;
    const int64_t pos = (int64_t)pb * 64 + 32 * grp + j;
    const int64_t r = pos - off;
    const bool active = r >= 0 && r < wk.q_len;

    const uint16_t* kbase = wk.kbase;
    const uint16_t* vbase = wk.vbase;
    const int64_t kv_len = wk.kv_len;
    const int T = pb;  // the diagonal tile, the last one

    StagePlan<PaddedTile, kPrefillWaves> plan;
    stage_plan(plan, lane, w);
    stage_tile(plan, kbase, vbase, 0, kv_len, smem, lane, w);
    if (T >= 1) stage_tile(plan, kbase, vbase, kTile, kv_len, smem + PaddedTile::kBytes, lane, w);

    const int64_t qrow0 = (int64_t)(w & 3) * wk.q_hstride;  // this wave's query head
    bf16x8 qf[8];
    {
        const uint16_t* qrow = wk.q0 + (qrow0 + (active ? r : 0)) * kHeadDim;
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const u32x4 x4 = *reinterpret_cast<const u32x4*>(qrow + 16 * st + 8 * h);  // row valid either way
            qf[st] = __builtin_bit_cast(bf16x8, active ? x4 : zero);
        }
    }

    // running maxima are kept in log2 units (max * c)
    float Mc = -__builtin_inff(), L = 0.0f;
    f32x16 O[4];
    float mc = -__builtin_inff(), l = 0.0f;
    f32x16 acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        O[db] = zero16();
        acc[db] = zero16();
    }
    bool have_total = false;
    auto close_chunk = [&]() {
        if (!have_total) {
            Mc = mc;
            L = l;
#pragma unroll
            for (int db = 0; db < 4; ++db) O[db] = acc[db];
            have_total = true;
        } else {
            float Mcn, A, B;
            fold_scalars(Mc, mc, Mcn, A, B);
            L = __builtin_fmaf(L, A, l * B);
#pragma unroll
            for (int db = 0; db < 4; ++db) {
#pragma unroll
                for (int v = 0; v < 16; ++v) O[db][v] = fold_value(O[db][v], A, acc[db][v], B);
            }
            Mc = Mcn;
        }
        mc = -__builtin_inff();
        l = 0.0f;
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[db] = zero16();
    };

    // Start of tile t's products: this wave's loads of tile t are done (group
    // 0 may still have those of tile t + 1 in flight, group 1 has not issued
    // them yet), then the barrier.
    auto tile_start = [&](int t) {
        if (t <= T) {
            if (t + 1 <= T && grp == 0)
                wait_stage_loads<PaddedTile, kPrefillWaves>(w);
            else
                wait_vm<0>();
        }
        __syncthreads();
    };
    f32x16 s0, s1;
    bf16x8 pf[2][2];
    float a_pend = 1.0f;  // rescale factor of the tile whose row sum is still to be added
    auto products = [&](int t) {
        __builtin_amdgcn_s_setprio(3);
        if (t >= 1) {
            float rs = 0.0f;
            pv_fenced_rs<PaddedTile, 4>(pf, smem + ((t - 1) % kStages) * PaddedTile::kBytes + PaddedTile::kKStage, lane,
                                        acc, 0, rs);
            float ls_lo, ls_hi;
            halves(rs, ls_lo, ls_hi);
            l = __builtin_fmaf(l, a_pend, ls_lo + ls_hi);
        }
        if (t <= T) qk_fenced<PaddedTile>(qf, smem + (t % kStages) * PaddedTile::kBytes, lane, s0, s1);
    };
    // the softmax of tile t < T; `first` on the first tile of a chunk
    auto softmax = [&](int t, bool first) {
        __builtin_amdgcn_s_setprio(0);
        if (t + 2 <= T)
            stage_tile(plan, kbase, vbase, (int64_t)(t + 2) * kTile, kv_len,
                       smem + ((t + 2) % kStages) * PaddedTile::kBytes, lane, w);
        softmax_tile<4, false>(s0, s1, lane, (int64_t)t * kTile, pos, c, mc, a_pend, acc, pf, first);
    };
    auto softmax_diag = [&](bool first) {
        __builtin_amdgcn_s_setprio(0);
        softmax_tile<4, true>(s0, s1, lane, (int64_t)T * kTile, pos, c, mc, a_pend, acc, pf, first);
    };
    // tiles below the diagonal chunk by chunk (the first tile of a chunk
    // peeled: the previous chunk is closed before its softmax), then the
    // diagonal tile T and the P V products of T
    const bool diag_first = (T % kTilesPerChunk) == 0;
    if (grp == 0) {
        for (int t0 = 0; t0 < T; t0 += kTilesPerChunk) {
            const int tend = min(t0 + kTilesPerChunk, T);
            tile_start(t0);
            products(t0);
            if (t0 > 0) close_chunk();
            softmax(t0, true);
            for (int t = t0 + 1; t < tend; ++t) {
                tile_start(t);
                products(t);
                softmax(t, false);
            }
        }
        tile_start(T);
        products(T);
        if (diag_first && T > 0) close_chunk();
        softmax_diag(diag_first);
        tile_start(T + 1);
        products(T + 1);
    } else {
        tile_start(0);
        products(0);
        for (int t0 = 0; t0 < T; t0 += kTilesPerChunk) {
            const int tend = min(t0 + kTilesPerChunk, T);
            tile_start(t0 + 1);
            if (t0 > 0) close_chunk();
            softmax(t0, true);
            products(t0 + 1);
            for (int t = t0 + 1; t < tend; ++t) {
                tile_start(t + 1);
                softmax(t, false);
                products(t + 1);
            }
        }
        tile_start(T + 1);
        if (diag_first && T > 0) close_chunk();
        softmax_diag(diag_first);
        products(T + 1);
    }
    close_chunk();
    __builtin_amdgcn_s_setprio(0);

    // The quotients of this lane's row, 4 columns per 8-byte piece: piece
    // (db, b4) holds columns 32 db + 8 b4 + 4 h .. + 3.  Swapping halves of
    // the wave between the pieces of b4 = 2m and 2m + 1 gives every lane the
    // 8 adjacent columns 32 db + 16 m + 8 h .. + 7, one 16-byte store.  The
    // swaps run in every lane (they read the partner lane), the stores only
    // in the active ones.
    {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                uint32_t a[2], b[2];
#pragma unroll
                for (int hv = 0; hv < 2; ++hv) {
                    const int va = 4 * (2 * m) + 2 * hv, vb = 4 * (2 * m + 1) + 2 * hv;
                    a[hv] = finalize(O[db][va], L) | ((uint32_t)finalize(O[db][va + 1], L) << 16);
                    b[hv] = finalize(O[db][vb], L) | ((uint32_t)finalize(O[db][vb + 1], L) << 16);
                }
                u32x4 out;
#pragma unroll
                for (int hv = 0; hv < 2; ++hv) {
                    // new first operand: lanes 32..63 take b of lanes 0..31;
                    // new second: lanes 0..31 take a of lanes 32..63
                    const auto sw = __builtin_amdgcn_permlane32_swap(a[hv], b[hv], false, false);
                    out[hv] = (uint32_t)sw[0];
                    out[2 + hv] = (uint32_t)sw[1];
                }
                if (active) *reinterpret_cast<u32x4*>(wk.o0 + (qrow0 + r) * kHeadDim + 32 * db + 16 * m + 8 * h) = out;
            }
        }
        if (active && wk.lse0 && h == 0) wk.lse0[qrow0 + r] = lse_of(Mc, L);
    }
}

// Work item x of a dense-batch launch (A: the launch's PrefillArgs, read
// from wherever the caller holds them).  Workgroups are dispatched to the 8
// XCDs round-robin (x % 8); when the (b, g) pairs split evenly over the
// XCDs, XCD k takes the pairs k, k + 8, ... one after another, each pair's
// position blocks longest first, so the blocks running together on an XCD
// stream the same K/V tiles through its L2.
template <class A>
__device__ __forceinline__ void prefill_item(const A& a, int x, PrefillWork& wk) {
    const int nbg = a.batch * a.n_kv_heads;
    int bg, pbr;
    if ((nbg & 7) == 0) {
        const int i = x >> 3;
        bg = (i / a.n_pb) * 8 + (x & 7);
        pbr = i % a.n_pb;
    } else {
        bg = x % nbg;
        pbr = x / nbg;
    }
    const int b = bg / a.n_kv_heads, g = bg % a.n_kv_heads;
    const int n_q_heads = kGroup * a.n_kv_heads;
    wk.q0 = a.q + ((int64_t)b * n_q_heads + kGroup * g) * a.q_len * kHeadDim;
    wk.o0 = a.o + ((int64_t)b * n_q_heads + kGroup * g) * a.q_len * kHeadDim;
    wk.lse0 = a.lse ? a.lse + ((int64_t)b * n_q_heads + kGroup * g) * a.q_len : nullptr;
    wk.q_hstride = a.q_len;
    const int64_t kvoff = ((int64_t)b * a.n_kv_heads + g) * a.cap * kHeadDim;
    wk.kbase = a.k + kvoff;
    wk.vbase = a.v + kvoff;
    wk.q_len = a.q_len;
    wk.kv_len = a.kv_len;
    wk.pb = a.pb_first + a.n_pb - 1 - pbr;
}

// Dense batch: q, o [batch, Hq, q_len, 128]; k, v [batch, Hkv, cap, 128].
// One workgroup per work item.
template <bool kPartitioned>
__global__ __launch_bounds__(64 * kPrefillWaves) void prefill_kernel(PrefillArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[kStages * PaddedTile::kBytes];
    PrefillWork wk;
    prefill_item(a, blockIdx.x, wk);
    prefill_body<kPartitioned>(wk, a.c, smem);
}

// The same work items, run by 8 U resident workgroups (one per CU: the LDS
// ring fills a CU) that each walk a fixed list, which saves the launch of a
// workgroup per item where items are few per CU.  Workgroup p sits on XCD
// k = p % 8 with local index u = p / 8 and takes XCD k's items x = 8 i + k
// in rounds of U: in round n, i = n U + u for even n and n U + U - 1 - u for
// odd n, so that two consecutive rounds give every workgroup the same number
// of tiles when the launch admits it (the launcher checks).  A barrier
// between items keeps the next item's first loads from reaching ring stages
// that the slower wave group still reads.  The arguments are read from the
// kernel-argument segment (PrefillArgs is the first argument, at offset 0)
// at each item, through a pointer the compiler cannot see as invariant, so
// that they hold no scalar registers across an item's tiles.
template <bool kPartitioned>
__global__ __launch_bounds__(64 * kPrefillWaves) void prefill_persistent_kernel(PrefillArgs a, int n_items) {
    __shared__ __attribute__((aligned(1024))) char smem[kStages * PaddedTile::kBytes];
    const int k = blockIdx.x & 7, u = blockIdx.x >> 3, U = gridDim.x >> 3;
    const int n_k = (n_items - k + 7) >> 3;  // items x < n_items with x % 8 == k
    for (int n = 0;; ++n) {
        const int i = n * U + ((n & 1) ? U - 1 - u : u);
        if (i >= n_k) break;
        uint64_t args = (uint64_t)(uintptr_t)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(args));
        PrefillWork wk;
        prefill_item(*reinterpret_cast<const __attribute__((address_space(4))) PrefillArgs*>(args), 8 * i + k, wk);
        if (n > 0) __syncthreads();
        prefill_body<kPartitioned>(wk, a.c, smem);
    }
}

// Ragged batch: the sequences of one launch (at most kMaxVarlenSeqs), packed
// head-major: q, o [Hq, q_rows, 128]; k, v [Hkv, kv_rows, 128].  Sequence s
// holds query rows q_row0[s] .. + q_len[s] - 1 and keys kv_row0[s] .. +
// kv_len[s] - 1; its row r sits at position kv_len[s] - q_len[s] + r.
constexpr int kMaxVarlenSeqs = 64;
struct VarlenTable {
    int64_t q_row0[kMaxVarlenSeqs];
    int64_t kv_row0[kMaxVarlenSeqs];
    int32_t q_len[kMaxVarlenSeqs];
    int32_t kv_len[kMaxVarlenSeqs];
    int32_t unit0[kMaxVarlenSeqs + 1];  // first work unit of each sequence (prefix sum)
    int32_t n_seqs;
};

struct VarlenArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;               // optional: [Hq, q_rows] log-sum-exp of each row
    int64_t q_rows, kv_rows;  // rows per head of the packed tensors
    int32_t n_kv_heads;
    float c;
};

// Work units of a sequence: (64-position block, KV head), longest blocks
// first.  All rows use the partitioned form (q_len == kv_len gives position r).
__global__ __launch_bounds__(64 * kPrefillWaves) void prefill_varlen_kernel(VarlenArgs a, VarlenTable t) {
    __shared__ __attribute__((aligned(1024))) char smem[kStages * PaddedTile::kBytes];
    const int x = blockIdx.x;
    int s = 0;
    while (s + 1 < t.n_seqs && t.unit0[s + 1] <= x) ++s;
    const int u = x - t.unit0[s];
    const int g = u % a.n_kv_heads, pbr = u / a.n_kv_heads;
    const int64_t q_len = t.q_len[s], kv_len = t.kv_len[s];
    PrefillWork wk;
    wk.q0 = a.q + ((int64_t)kGroup * g * a.q_rows + t.q_row0[s]) * kHeadDim;
    wk.o0 = a.o + ((int64_t)kGroup * g * a.q_rows + t.q_row0[s]) * kHeadDim;
    wk.lse0 = a.lse ? a.lse + (int64_t)kGroup * g * a.q_rows + t.q_row0[s] : nullptr;
    wk.q_hstride = a.q_rows;
    wk.kbase = a.k + ((int64_t)g * a.kv_rows + t.kv_row0[s]) * kHeadDim;
    wk.vbase = a.v + ((int64_t)g * a.kv_rows + t.kv_row0[s]) * kHeadDim;
    wk.q_len = q_len;
    wk.kv_len = kv_len;
    wk.pb = (int)((kv_len - 1) / 64) - pbr;
    prefill_body<true>(wk, a.c, smem);
}

struct DecodeArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* ws_o;   // [batch * n_q_heads * n_chunks][128]
    float* ws_ml;  // [batch * n_q_heads * n_chunks][2]: (max * c, sum)
    float* lse;    // optional: [batch, Hq, n_rows] log-sum-exp of each row
    int64_t kv_len, cap;
    int32_t batch, n_kv_heads, n_chunks;
    int32_t n_rows;  // query rows per head (1 = one-token decode, at most kDecodeMaxRows)
    float c;
};

constexpr int kDecodeWaves = 4;
// query rows per head a decode workgroup can carry: 4 heads x 8 rows fill the
// 32 columns of one MFMA block
constexpr int kDecodeMaxRows = 8;
// K and V are loaded kDecodeLead iterations before they are read
// (decode_body); the rings take 2 (kDecodeLead + 1) x 16 KiB of LDS.  With
// one iteration of lead (64 KiB) two workgroups share a CU; deeper leads
// (96 and 128 KiB, one workgroup per CU) measured slower at every batch.
constexpr int kDecodeLead = 1;
constexpr int kDecodeLdsBytes = 2 * (kDecodeLead + 1) * SwizzledTile::kKStage;

// Everything a decode workgroup needs once its work item is known.
struct DecodeWork {
    const uint16_t* q;  // query head 4g + i, row r at row q_row0 + i * q_hstride + r
    uint16_t* o;        // output rows, same indexing
    float* lse;         // optional log-sum-exp output, same row indexing
    int64_t q_row0, q_hstride;
    int n_rows;         // query rows per head, at positions kv_len - n_rows .. kv_len - 1
    const uint16_t* kbase;  // key 0 of this (sequence, KV head)
    const uint16_t* vbase;
    int64_t kv_len;
    int chunk, n_chunks;
    int64_t ws_row0;  // partial of query head 4g + i, row r, this chunk: ws row ws_row0 + (i n_rows + r) n_chunks + chunk
    // paged caches only: this sequence's row of the block table and the pool
    const int32_t* pages;
    const uint16_t* kpool;
    const uint16_t* vpool;
    int64_t page_elems;  // elements of one page (all KV heads)
    int64_t head_elems;  // offset of this KV head inside a page
    int32_t page_size, n_pages;
};

// Workgroup = 4 waves on one (sequence, KV head, chunk).  The four query heads
// sit in MFMA columns 0..3 (the other columns hold zeros).  Every wave computes
// the scores of the tile; wave w accumulates the output rows d = 32w..32w+31.
// The chunk's tiles stream through LDS rings of K and V, and the scores of
// tile t + 1 are computed beside the softmax and P V of tile t (the same
// operations as tile_step, so the bits of the prefill).  With kPaged
// the keys come from a paged cache: a page holds page_size (a multiple of 64)
// consecutive keys, so every 64-key tile lies inside one page; page indices
// are clamped to the pool, so no table entry can make a load leave it.
template <bool kPaged, int kLead>
__device__ __forceinline__ void decode_body(const DecodeWork& wk, float* ws_o, float* ws_ml, float c, char* smem) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int chunk = wk.chunk;
    const int j = lane & 31, h = lane >> 5;
    const int n_rows = wk.n_rows;
    // MFMA column j = query head 4g + hi, row ri (columns beyond 4 n_rows hold zeros)
    const bool col = j < kGroup * n_rows;
    const int hi = col ? j / n_rows : 0;
    const int ri = col ? j % n_rows : 0;
    const int64_t kv_len = wk.kv_len;
    const int64_t pos = kv_len - n_rows + ri;

    const uint16_t* kbase = wk.kbase;
    const uint16_t* vbase = wk.vbase;
    const int n_tiles = (int)((kv_len + kTile - 1) / kTile);
    const int t0 = chunk * kTilesPerChunk;
    const int t1 = min(t0 + kTilesPerChunk, n_tiles);
    // a row takes part in the chunks up to the one holding its position; in a
    // later chunk every key is masked for it and its column is not stored
    const bool active = col && pos >= (int64_t)t0 * kTile;

    StagePlan<SwizzledTile, kDecodeWaves> plan;
    stage_plan(plan, lane, w);

    // paged: lane i holds the pool index of the chunk's i-th page (at most 16)
    int pg = 0, p0 = 0;
    if (kPaged) {
        p0 = (int)((int64_t)t0 * kTile / wk.page_size);
        const int p1 = (int)((min((int64_t)t1 * kTile, kv_len) - 1) / wk.page_size);
        pg = lane <= p1 - p0 ? wk.pages[p0 + lane] : 0;
        pg = min(max(pg, 0), wk.n_pages - 1);
    }
    // K and V stream through separate rings of kLead + 1 stages of 16 KiB:
    // the scores of tile t + 1 read K(t + 1) while the P V products of tile t
    // read V(t).  Iteration t starts, after a barrier, the pair
    // (K(t + kLead + 1), V(t + kLead)) into the stages of K(t) and V(t - 1),
    // which every wave has finished with; the pair is needed kLead
    // iterations later.
    constexpr int kKStages = kLead + 1, kVStages = kLead + 1;
    char* const kring = smem;
    char* const vring = smem + kKStages * SwizzledTile::kKStage;
    auto kst = [&](int t) { return kring + (t % kKStages) * SwizzledTile::kKStage; };
    auto vst = [&](int t) { return vring + (t % kVStages) * SwizzledTile::kKStage; };
    auto tile_base = [&](int t, const uint16_t* pool, const uint16_t* dense, int64_t& key0, int64_t& len) {
        key0 = (int64_t)t * kTile;
        len = kv_len;
        if (kPaged) {
            const int page = __builtin_amdgcn_readlane(pg, (int)(key0 / wk.page_size) - p0);
            const int64_t off = (int64_t)page * wk.page_elems + wk.head_elems + (key0 % wk.page_size) * kHeadDim;
            len = min((int64_t)kTile, kv_len - key0);
            key0 = 0;
            return pool + off;
        }
        return dense;
    };
    auto load_k = [&](int t) {
        int64_t key0, len;
        const uint16_t* base = tile_base(t, wk.kpool, kbase, key0, len);
        stage_half<SwizzledTile, kDecodeWaves, false>(plan, base, key0, len, kst(t), lane, w);
    };
    auto load_v = [&](int t) {
        int64_t key0, len;
        const uint16_t* base = tile_base(t, wk.vpool, vbase, key0, len);
        stage_half<SwizzledTile, kDecodeWaves, true>(plan, base, key0, len, vst(t), lane, w);
    };
    // the pair of iteration s (s < t0: issued before the loop)
    constexpr int kHalfLoads = SwizzledTile::kKLoads / kDecodeWaves;  // per wave and half tile
    auto pair_loads = [&](int s) { return (s + kLead + 1 < t1 ? kHalfLoads : 0) + (s + kLead < t1 ? kHalfLoads : 0); };
    auto issue_pair = [&](int s) {
        if (s + kLead + 1 < t1) load_k(s + kLead + 1);
        if (s + kLead < t1) load_v(s + kLead);
    };
    // wait until at most `allow` of this wave's loads are pending
    auto wait_allow = [&](int allow) {
        switch (allow / kHalfLoads) {
            case 0: wait_vm<0>(); break;
            case 1: wait_vm<kHalfLoads>(); break;
            case 2: wait_vm<2 * kHalfLoads>(); break;
            case 3: wait_vm<3 * kHalfLoads>(); break;
            case 4: wait_vm<4 * kHalfLoads>(); break;
            case 5: wait_vm<5 * kHalfLoads>(); break;
            default: wait_vm<6 * kHalfLoads>(); break;
        }
    };
    static_assert(kLead >= 1 && kLead <= 4, "wait_allow covers the loads of up to three pairs");

    const int64_t qrow_idx = wk.q_row0 + (int64_t)hi * wk.q_hstride + ri;
    bf16x8 qf[8];
    {
        const uint16_t* qrow = wk.q + qrow_idx * kHeadDim;
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const u32x4 x4 = *reinterpret_cast<const u32x4*>(qrow + 16 * st + 8 * h);  // row valid either way
            qf[st] = __builtin_bit_cast(bf16x8, active ? x4 : zero);
        }
    }

    // Q first, then K(t0) and the pairs of iterations t0 - kLead .. t0 - 1
    load_k(t0);
    for (int s = t0 - kLead; s < t0; ++s) issue_pair(s);
    float mc = -__builtin_inff(), l = 0.0f;  // max in log2 units
    f32x16 acc[1];
    acc[0] = zero16();
    // (the first use of the Q fragments waits for every load issued so far)
    wait_vm<0>();
    __syncthreads();
    f32x16 s0, s1;
    qk_plain<SwizzledTile>(qf, kst(t0), lane, s0, s1);
    // Tiles from t_mask on hold keys beyond the first row's position (only
    // the context's last tile when n_rows = 1) and take the masked softmax.
    // The scores of tile t + 1 are computed in iteration t even past the
    // chunk's end (from a stale or unwritten stage; never used), which keeps
    // each iteration one straight block.
    const int64_t full = kv_len - n_rows - (kTile - 1);  // tile t is unmasked iff 64 t <= full and t < n_tiles - 1
    const int t_mask = full < 0 ? 0 : min(n_tiles - 1, (int)(full / kTile) + 1);
    auto iteration = [&](int t, auto masked) {
        // K(t + 1) and V(t) came with the pair of iteration t - kLead; the
        // pairs of the iterations after it may still be in flight
        int allow = 0;
        for (int s = t - kLead + 1; s < t; ++s) allow += pair_loads(s);
        wait_allow(allow);
        __syncthreads();
        issue_pair(t);
        bf16x8 pf[2][2];
        softmax_flat<1, decltype(masked)::value>(s0, s1, lane, (int64_t)t * kTile, pos, c, mc, l, acc, pf);
        f32x16 n0, n1;
        qk_plain<SwizzledTile>(qf, kst(t + 1), lane, n0, n1);
        pv_plain<SwizzledTile, 1>(pf, vst(t), lane, acc, w);
        s0 = n0;
        s1 = n1;
    };
    int t = t0;
    for (; t < min(t1, t_mask); ++t) iteration(t, std::false_type{});
    for (; t < t1; ++t) iteration(t, std::true_type{});

    if (!active) return;
    if (wk.n_chunks == 1) {
        // a single chunk is copied into the total: out = o / l
        uint16_t* orow = wk.o + qrow_idx * kHeadDim;
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
            const uint32_t e0 = finalize(acc[0][4 * b4 + 0], l), e1 = finalize(acc[0][4 * b4 + 1], l);
            const uint32_t e2 = finalize(acc[0][4 * b4 + 2], l), e3 = finalize(acc[0][4 * b4 + 3], l);
            uint2 packed;
            packed.x = e0 | (e1 << 16);
            packed.y = e2 | (e3 << 16);
            *reinterpret_cast<uint2*>(orow + 32 * w + 8 * b4 + 4 * h) = packed;
        }
        if (wk.lse && w == 0 && h == 0) wk.lse[qrow_idx] = lse_of(mc, l);
        return;
    }
    const int64_t prow = wk.ws_row0 + ((int64_t)hi * n_rows + ri) * wk.n_chunks + chunk;
    float* po = ws_o + prow * kHeadDim;
#pragma unroll
    for (int b4 = 0; b4 < 4; ++b4) {
        float4 f;
        f.x = acc[0][4 * b4 + 0];
        f.y = acc[0][4 * b4 + 1];
        f.z = acc[0][4 * b4 + 2];
        f.w = acc[0][4 * b4 + 3];
        *reinterpret_cast<float4*>(po + 32 * w + 8 * b4 + 4 * h) = f;
    }
    if (w == 0 && h == 0) {
        ws_ml[prow * 2 + 0] = mc;
        ws_ml[prow * 2 + 1] = l;
    }
}

// Dense batch: q, o [batch, Hq, 1, 128]; caches [batch, Hkv, cap, 128].
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[kDecodeLdsBytes];
    const int x = blockIdx.x;
    const int chunk = x % a.n_chunks;
    const int bg = x / a.n_chunks;
    const int b = bg / a.n_kv_heads, g = bg % a.n_kv_heads;
    const int n_q_heads = kGroup * a.n_kv_heads;
    DecodeWork wk;
    wk.q = a.q;
    wk.o = a.o;
    wk.lse = a.lse;
    wk.q_row0 = ((int64_t)b * n_q_heads + kGroup * g) * a.n_rows;
    wk.q_hstride = a.n_rows;
    wk.n_rows = a.n_rows;
    const int64_t kvoff = ((int64_t)b * a.n_kv_heads + g) * a.cap * kHeadDim;
    wk.kbase = a.k + kvoff;
    wk.vbase = a.v + kvoff;
    wk.kv_len = a.kv_len;
    wk.chunk = chunk;
    wk.n_chunks = a.n_chunks;
    wk.ws_row0 = wk.q_row0 * a.n_chunks;
    decode_body<false, kDecodeLead>(wk, a.ws_o, a.ws_ml, a.c, smem);
}

struct CombineArgs {
    const float* ws_o;
    const float* ws_ml;
    uint16_t* o;
    float* lse;  // optional: [rows] log-sum-exp
    int64_t kv_len;
    int32_t n_chunks;
    int32_t n_rows;  // rows per head: output row R is row R % n_rows of its head
    float c;
};

// Fold the chunk partials of one output row in chunk order and finalize;
// thread d owns output element d; thread 0 writes the log-sum-exp when asked.
__device__ __forceinline__ void combine_row(const float* ws_o, const float* ws_ml, int64_t base, int n_chunks,
                                            uint16_t* orow, float* lse_row) {
    const int d = threadIdx.x;
    // partials are loaded kBatch chunks at a time (chunk 0 with the first
    // batch), then folded one by one in chunk order, so the loads of a batch
    // are in flight together; chunk 0 is the total the others fold into
    constexpr int kBatch = 8;
    float Mc = 0.0f, L = 0.0f, O = 0.0f;
    for (int k0 = 0; k0 < n_chunks; k0 += kBatch) {
        float mcs[kBatch], ls[kBatch], os[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int64_t r = base + min(k0 + i, n_chunks - 1);
            mcs[i] = ws_ml[r * 2 + 0];
            ls[i] = ws_ml[r * 2 + 1];
            os[i] = ws_o[r * kHeadDim + d];
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            if (k0 + i == 0) {
                Mc = mcs[0];
                L = ls[0];
                O = os[0];
            } else if (k0 + i < n_chunks) {
                float Mcn, A, B;
                fold_scalars(Mc, mcs[i], Mcn, A, B);
                L = __builtin_fmaf(L, A, ls[i] * B);
                O = fold_value(O, A, os[i], B);
                Mc = Mcn;
            }
        }
    }
    orow[d] = finalize(O, L);
    if (lse_row && d == 0) *lse_row = lse_of(Mc, L);
}

__global__ __launch_bounds__(128) void combine_kernel(CombineArgs a) {
    const int64_t row = blockIdx.x;
    // the row's chunks: those up to the one holding its position
    const int64_t pos = a.kv_len - a.n_rows + row % a.n_rows;
    const int nc = (int)(pos / kChunk) + 1;
    combine_row(a.ws_o, a.ws_ml, row * a.n_chunks, nc, a.o + row * kHeadDim, a.lse ? a.lse + row : nullptr);
}

// Ragged decode: one query token per sequence, q, o [Hq, n_seq_total, 128]
// packed head-major; caches [Hkv, kv_rows, 128] with sequence s's keys at
// rows kv_row0[s] .. + kv_len[s] - 1.  Work units of a sequence: (KV head,
// chunk); its partials start at workspace row ws_row0[s] (Hq * n_chunks rows).
struct DecodeVarlenTable {
    int64_t kv_row0[kMaxVarlenSeqs];
    int64_t ws_row0[kMaxVarlenSeqs];
    int32_t kv_len[kMaxVarlenSeqs];
    int32_t seq[kMaxVarlenSeqs];        // the sequence's index among all query tokens
    int32_t unit0[kMaxVarlenSeqs + 1];  // first work unit of each sequence (prefix sum)
    int32_t n_seqs;
};

struct DecodeVarlenArgs {
    const uint16_t* q;
    const uint16_t* k;  // packed caches, or the page pools (paged)
    const uint16_t* v;
    uint16_t* o;
    float* ws_o;
    float* ws_ml;
    int64_t tok_stride, head_stride;  // query / output row of (sequence s, head h): s * tok_stride + h * head_stride
    int64_t kv_rows;                  // packed caches: rows per KV head
    const int32_t* block_table;       // paged: [sequences, max_pages] pool indices
    int64_t max_pages;
    int32_t page_size, n_pages;
    int32_t n_kv_heads;
    float c;
};

template <bool kPaged>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_varlen_kernel(DecodeVarlenArgs a, DecodeVarlenTable t) {
    __shared__ __attribute__((aligned(1024))) char smem[kDecodeLdsBytes];
    const int x = blockIdx.x;
    int s = 0;
    while (s + 1 < t.n_seqs && t.unit0[s + 1] <= x) ++s;
    const int64_t kv_len = t.kv_len[s];
    const int nc = (int)((kv_len + kChunk - 1) / kChunk);
    const int u = x - t.unit0[s];
    const int g = u / nc, chunk = u % nc;
    DecodeWork wk;
    wk.q = a.q;
    wk.o = a.o;
    wk.lse = nullptr;
    wk.q_row0 = (int64_t)t.seq[s] * a.tok_stride + (int64_t)kGroup * g * a.head_stride;
    wk.q_hstride = a.head_stride;
    wk.n_rows = 1;
    if (kPaged) {
        wk.kbase = wk.vbase = nullptr;
        wk.pages = a.block_table + (int64_t)t.seq[s] * a.max_pages;
        wk.kpool = a.k;
        wk.vpool = a.v;
        wk.page_elems = (int64_t)a.n_kv_heads * a.page_size * kHeadDim;
        wk.head_elems = (int64_t)g * a.page_size * kHeadDim;
        wk.page_size = a.page_size;
        wk.n_pages = a.n_pages;
    } else {
        wk.kbase = a.k + ((int64_t)g * a.kv_rows + t.kv_row0[s]) * kHeadDim;
        wk.vbase = a.v + ((int64_t)g * a.kv_rows + t.kv_row0[s]) * kHeadDim;
    }
    wk.kv_len = kv_len;
    wk.chunk = chunk;
    wk.n_chunks = nc;
    wk.ws_row0 = t.ws_row0[s] + (int64_t)kGroup * g * nc;
    decode_body<kPaged, kDecodeLead>(wk, a.ws_o, a.ws_ml, a.c, smem);
}

// One workgroup per (sequence with more than one chunk, query head).
__global__ __launch_bounds__(128) void combine_varlen_kernel(DecodeVarlenArgs a, DecodeVarlenTable t) {
    const int n_q_heads = kGroup * a.n_kv_heads;
    const int s = blockIdx.x / n_q_heads, head = blockIdx.x % n_q_heads;
    const int64_t kv_len = t.kv_len[s];
    const int nc = (int)((kv_len + kChunk - 1) / kChunk);
    if (nc == 1) return;
    combine_row(a.ws_o, a.ws_ml, t.ws_row0[s] + (int64_t)head * nc, nc,
                a.o + ((int64_t)t.seq[s] * a.tok_stride + (int64_t)head * a.head_stride) * kHeadDim, nullptr);
}

}  // namespace kb

// Partials of kb_attn_decode_static (for callers that cannot allocate): one
// copy per GPU, held until the process ends.  Host code never uses this name
// as an address; it looks up each device's copy (static_scratch below).
static __device__ __align__(256) float scratch[KB_ATTN_DECODE_STATIC_SCRATCH_BYTES / sizeof(float)];

namespace kb {

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

constexpr int64_t kMaxLen = int64_t(1) << 30;  // positions stay in int32 tile arithmetic

float contract_c(float scale) { return (float)((double)scale * 1.4426950408889634073599246810019); }

bool ranges_overlap(const void* a, size_t an, const void* b, size_t bn) {
    if (!a || !b || !an || !bn) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

int check_heads(int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim) {
    if (n_q_heads < 1 || n_kv_heads < 1 || head_dim < 1) return KB_ATTN_ERR_INVALID_ARG;
    if (head_dim != kHeadDim || n_q_heads != kGroup * n_kv_heads) return KB_ATTN_ERR_UNSUPPORTED;
    return KB_ATTN_OK;
}

int check_scale(float scale) {
    return (std::isfinite(scale) && scale > 0.0f) ? KB_ATTN_OK : KB_ATTN_ERR_INVALID_ARG;
}

int check_aligned(std::initializer_list<const void*> ptrs) {
    for (const void* p : ptrs)
        if (p && ((uintptr_t)p & 15u)) return KB_ATTN_ERR_ALIGNMENT;
    return KB_ATTN_OK;
}

int check_device(std::initializer_list<const void*> ptrs) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return KB_ATTN_ERR_DEVICE;
    }
    for (const void* p : ptrs) {
        if (!p) continue;
        hipPointerAttribute_t attr;
        if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
            (void)hipGetLastError();
            return KB_ATTN_ERR_DEVICE;
        }
        if (attr.type != hipMemoryTypeDevice || attr.device != dev) return KB_ATTN_ERR_DEVICE;
    }
    return KB_ATTN_OK;
}

int64_t n_chunks_of(int64_t kv_len) { return (kv_len + kChunk - 1) / kChunk; }

// Device address of the current device's copy of `scratch`, looked up once
// per device (hipGetSymbolAddress with that device current) and kept.
constexpr int kMaxDevices = 64;
int static_scratch(void** out) {
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return KB_ATTN_ERR_DEVICE;
    }
    if (dev < 0 || dev >= kMaxDevices) return KB_ATTN_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return KB_ATTN_ERR_HIP;
        }
        addr[dev] = p;
    }
    *out = addr[dev];
    return KB_ATTN_OK;
}

// CUs of the current device when their number is a multiple of the 8 XCDs,
// else 0; looked up once per device and kept.
int resident_prefill_workgroups() {
    static std::mutex mu;
    static int cus[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return 0;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
            (void)hipGetLastError();
            n = 0;
        }
        cus[dev] = (n > 0 && n % 8 == 0) ? n : -1;
    }
    return cus[dev] > 0 ? cus[dev] : 0;
}

// The persistent prefill runs when its fixed schedule balances and pays: the
// (b, g) pairs split evenly over the XCDs, each XCD's item count is a whole
// number of round pairs, and a pair's position blocks either fill whole
// round pairs or divide a round (then every two consecutive rounds give each
// workgroup the same tiles); and there are 2 to 16 items per workgroup (with
// more, the launch cost it saves is a smaller share than the balance the
// hardware's own dispatch keeps: measured slower at 128 per workgroup).
bool use_persistent_prefill(const PrefillArgs& a, int64_t n_items, int resident) {
    if (resident <= 0) return false;
    const int64_t U = resident / 8, nbg = (int64_t)a.batch * a.n_kv_heads;
    if (nbg % 8 != 0 || n_items < 2 * (int64_t)resident || n_items > 16 * (int64_t)resident) return false;
    if ((n_items / 8) % (2 * U) != 0) return false;
    return a.n_pb % (2 * U) == 0 || U % a.n_pb == 0;
}

int launch_prefill(bool partitioned, const void* q, const void* k, const void* v, void* o, float* lse,
                   int64_t batch, int64_t q_len, int64_t kv_len, int64_t cap, int32_t n_kv_heads, float scale,
                   hipStream_t stream) {
    PrefillArgs a;
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.o = (uint16_t*)o;
    a.lse = lse;
    a.q_len = q_len;
    a.kv_len = kv_len;
    a.cap = cap;
    a.batch = (int32_t)batch;
    a.n_kv_heads = n_kv_heads;
    const int64_t first = (kv_len - q_len) / 64, last = (kv_len - 1) / 64;
    a.pb_first = (int32_t)first;
    a.n_pb = (int32_t)(last - first + 1);
    a.c = contract_c(scale);
    const int64_t grid = (int64_t)a.n_pb * batch * n_kv_heads;
    if (grid > INT32_MAX) return KB_ATTN_ERR_LENGTH;
    const int resident = resident_prefill_workgroups();
    if (use_persistent_prefill(a, grid, resident)) {
        if (!partitioned)
            hipLaunchKernelGGL(prefill_persistent_kernel<false>, dim3((unsigned)resident), dim3(64 * kPrefillWaves), 0,
                               stream, a, (int)grid);
        else
            hipLaunchKernelGGL(prefill_persistent_kernel<true>, dim3((unsigned)resident), dim3(64 * kPrefillWaves), 0,
                               stream, a, (int)grid);
    } else if (!partitioned) {
        hipLaunchKernelGGL(prefill_kernel<false>, dim3((unsigned)grid), dim3(64 * kPrefillWaves), 0, stream, a);
    } else {
        hipLaunchKernelGGL(prefill_kernel<true>, dim3((unsigned)grid), dim3(64 * kPrefillWaves), 0, stream, a);
    }
    return hipGetLastError() == hipSuccess ? KB_ATTN_OK : KB_ATTN_ERR_HIP;
}

// One sequence of a ragged call, after validation.
struct RaggedSeq {
    int64_t index;          // position in the caller's arrays
    int64_t q_row0, q_len;  // query rows in the packed q / o
    int64_t kv_row0, kv_len;
};

// Reads a ragged call's host arrays: query offsets cu_q (batch + 1 entries,
// non-decreasing), cache offsets cu_kv (same), and, when given, the number of
// valid keys of each sequence (else the whole cache range).  Checks every
// sequence against the contract's rules (0 <= q_len <= kv_len <= capacity,
// and kv_len >= 1 when q_len >= 1) before anything is launched.
int read_ragged(const int64_t* cu_q, const int64_t* cu_kv, const int64_t* kv_lens, int64_t batch,
                std::vector<RaggedSeq>& seqs, int64_t& q_rows, int64_t& kv_rows) {
    if (!cu_q || !cu_kv || batch < 1) return KB_ATTN_ERR_INVALID_ARG;
    if (cu_q[0] < 0 || cu_kv[0] < 0) return KB_ATTN_ERR_LENGTH;
    seqs.clear();
    for (int64_t i = 0; i < batch; ++i) {
        const int64_t q_len = cu_q[i + 1] - cu_q[i], cap = cu_kv[i + 1] - cu_kv[i];
        if (q_len < 0 || cap < 0) return KB_ATTN_ERR_LENGTH;
        const int64_t kv_len = kv_lens ? kv_lens[i] : cap;
        if (kv_len < 0 || kv_len > cap || q_len > kv_len || cap > kMaxLen) return KB_ATTN_ERR_LENGTH;
        if (q_len > 0) seqs.push_back({i, cu_q[i], q_len, cu_kv[i], kv_len});
    }
    q_rows = cu_q[batch];
    kv_rows = cu_kv[batch];
    if (q_rows > kMaxLen * 64 || kv_rows > kMaxLen * 64) return KB_ATTN_ERR_LENGTH;
    return KB_ATTN_OK;
}

int launch_prefill_varlen(const void* q, const void* k, const void* v, void* o, float* lse, std::vector<RaggedSeq> seqs,
                          int64_t q_rows, int64_t kv_rows, int32_t n_kv_heads, float scale, hipStream_t stream) {
    // longest sequences first, so the longest position blocks start first
    std::stable_sort(seqs.begin(), seqs.end(),
                     [](const RaggedSeq& x, const RaggedSeq& y) { return x.kv_len > y.kv_len; });
    VarlenArgs a;
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.o = (uint16_t*)o;
    a.lse = lse;
    a.q_rows = q_rows;
    a.kv_rows = kv_rows;
    a.n_kv_heads = n_kv_heads;
    a.c = contract_c(scale);
    for (size_t first = 0; first < seqs.size(); first += kMaxVarlenSeqs) {
        const size_t n = std::min(seqs.size() - first, (size_t)kMaxVarlenSeqs);
        VarlenTable t;
        t.n_seqs = (int32_t)n;
        int64_t units = 0;
        for (size_t i = 0; i < n; ++i) {
            const RaggedSeq& sq = seqs[first + i];
            t.q_row0[i] = sq.q_row0;
            t.kv_row0[i] = sq.kv_row0;
            t.q_len[i] = (int32_t)sq.q_len;
            t.kv_len[i] = (int32_t)sq.kv_len;
            t.unit0[i] = (int32_t)units;
            const int64_t n_pb = (sq.kv_len - 1) / 64 - (sq.kv_len - sq.q_len) / 64 + 1;
            units += n_pb * n_kv_heads;
            if (units > INT32_MAX) return KB_ATTN_ERR_LENGTH;
        }
        t.unit0[n] = (int32_t)units;
        hipLaunchKernelGGL(prefill_varlen_kernel, dim3((unsigned)units), dim3(64 * kPrefillWaves), 0, stream, a, t);
        if (hipGetLastError() != hipSuccess) return KB_ATTN_ERR_HIP;
    }
    return KB_ATTN_OK;
}

// Workspace rows (one per query head and chunk) of the ragged decode, for the
// sequences that have more than one chunk; ws_row0 gets each one's first row.
int64_t ragged_ws_rows(const std::vector<RaggedSeq>& seqs, int32_t n_q_heads, std::vector<int64_t>* ws_row0) {
    int64_t rows = 0;
    if (ws_row0) ws_row0->clear();
    for (const RaggedSeq& sq : seqs) {
        if (ws_row0) ws_row0->push_back(rows);
        const int64_t nc = n_chunks_of(sq.kv_len);
        if (nc > 1) rows += (int64_t)n_q_heads * nc;
    }
    return rows;
}

// Issue a ragged or paged decode: launches of at most kMaxVarlenSeqs
// sequences, each followed by its combine when a sequence has several chunks.
int launch_decode_tables(const DecodeVarlenArgs& a, const std::vector<RaggedSeq>& seqs,
                         const std::vector<int64_t>& ws_row0, int32_t n_q_heads, bool paged, hipStream_t stream) {
    for (size_t first = 0; first < seqs.size(); first += kMaxVarlenSeqs) {
        const size_t n = std::min(seqs.size() - first, (size_t)kMaxVarlenSeqs);
        DecodeVarlenTable t;
        t.n_seqs = (int32_t)n;
        int64_t units = 0;
        bool any_multi = false;
        for (size_t i = 0; i < n; ++i) {
            const RaggedSeq& sq = seqs[first + i];
            t.kv_row0[i] = sq.kv_row0;
            t.ws_row0[i] = ws_row0[first + i];
            t.kv_len[i] = (int32_t)sq.kv_len;
            t.seq[i] = (int32_t)sq.index;
            t.unit0[i] = (int32_t)units;
            const int64_t nc = n_chunks_of(sq.kv_len);
            any_multi = any_multi || nc > 1;
            units += nc * a.n_kv_heads;
            if (units > INT32_MAX) return KB_ATTN_ERR_LENGTH;
        }
        t.unit0[n] = (int32_t)units;
        if (paged)
            hipLaunchKernelGGL(decode_varlen_kernel<true>, dim3((unsigned)units), dim3(64 * kDecodeWaves), 0, stream, a,
                               t);
        else
            hipLaunchKernelGGL(decode_varlen_kernel<false>, dim3((unsigned)units), dim3(64 * kDecodeWaves), 0, stream,
                               a, t);
        if (hipGetLastError() != hipSuccess) return KB_ATTN_ERR_HIP;
        if (any_multi) {
            hipLaunchKernelGGL(combine_varlen_kernel, dim3((unsigned)(n * n_q_heads)), dim3(kHeadDim), 0, stream, a,
                               t);
            if (hipGetLastError() != hipSuccess) return KB_ATTN_ERR_HIP;
        }
    }
    return KB_ATTN_OK;
}

}  // namespace
}  // namespace kb

using namespace kb;

namespace {

// An optional log-sum-exp output of n_rows floats: 4-byte aligned device
// memory of the current device that overlaps none of the other buffers
// (alignment and overlap are checked before any device query).
int check_lse(const float* lse, size_t n_rows, std::initializer_list<std::pair<const void*, size_t>> others) {
    if (!lse) return KB_ATTN_OK;
    if ((uintptr_t)lse & 3u) return KB_ATTN_ERR_ALIGNMENT;
    for (const auto& o : others)
        if (ranges_overlap(lse, n_rows * sizeof(float), o.first, o.second)) return KB_ATTN_ERR_ALIAS;
    return check_device({lse});
}

int prefill_entry(const void* q, const void* k, const void* v, void* o, float* lse, int64_t batch, int64_t seq_len,
                  int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float scale, hipStream_t stream) {
    if (!q || !k || !v || !o || batch < 1 || seq_len < 1) return KB_ATTN_ERR_INVALID_ARG;
    if (int rc = check_heads(n_q_heads, n_kv_heads, head_dim)) return rc;
    if (int rc = check_scale(scale)) return rc;
    if (seq_len > kMaxLen || batch * n_kv_heads > INT32_MAX) return KB_ATTN_ERR_LENGTH;
    if (int rc = check_aligned({q, k, v, o})) return rc;
    const size_t qbytes = (size_t)batch * n_q_heads * seq_len * kHeadDim * 2;
    const size_t kvbytes = (size_t)batch * n_kv_heads * seq_len * kHeadDim * 2;
    if (ranges_overlap(o, qbytes, q, qbytes) || ranges_overlap(o, qbytes, k, kvbytes) ||
        ranges_overlap(o, qbytes, v, kvbytes))
        return KB_ATTN_ERR_ALIAS;
    if (int rc = check_lse(lse, (size_t)batch * n_q_heads * seq_len,
                           {{q, qbytes}, {k, kvbytes}, {v, kvbytes}, {o, qbytes}}))
        return rc;
    if (int rc = check_device({q, k, v, o})) return rc;
    return launch_prefill(false, q, k, v, o, lse, batch, seq_len, seq_len, seq_len, n_kv_heads, scale, stream);
}

int partitioned_entry(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int64_t batch,
                      int64_t q_len, int64_t kv_len, int64_t kv_capacity, int32_t n_q_heads, int32_t n_kv_heads,
                      int32_t head_dim, float scale, hipStream_t stream) {
    if (!q || !k_cache || !v_cache || !o || batch < 1) return KB_ATTN_ERR_INVALID_ARG;
    if (int rc = check_heads(n_q_heads, n_kv_heads, head_dim)) return rc;
    if (int rc = check_scale(scale)) return rc;
    if (q_len < 1 || q_len > kv_len || kv_len > kv_capacity) return KB_ATTN_ERR_LENGTH;
    if (kv_capacity > kMaxLen || batch * n_kv_heads > INT32_MAX) return KB_ATTN_ERR_LENGTH;
    if (int rc = check_aligned({q, k_cache, v_cache, o})) return rc;
    const size_t qbytes = (size_t)batch * n_q_heads * q_len * kHeadDim * 2;
    const size_t kvbytes = (size_t)batch * n_kv_heads * kv_capacity * kHeadDim * 2;
    if (ranges_overlap(o, qbytes, q, qbytes) || ranges_overlap(o, qbytes, k_cache, kvbytes) ||
        ranges_overlap(o, qbytes, v_cache, kvbytes))
        return KB_ATTN_ERR_ALIAS;
    if (int rc = check_lse(lse, (size_t)batch * n_q_heads * q_len,
                           {{q, qbytes}, {k_cache, kvbytes}, {v_cache, kvbytes}, {o, qbytes}}))
        return rc;
    if (int rc = check_device({q, k_cache, v_cache, o})) return rc;
    return launch_prefill(true, q, k_cache, v_cache, o, lse, batch, q_len, kv_len, kv_capacity, n_kv_heads, scale,
                          stream);
}

// With static_ws the partials go to the library's `scratch` array instead of
// a caller workspace (workspace and workspace_bytes are ignored).
int decode_entry(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int64_t batch,
                 int64_t n_rows, int64_t kv_len, int64_t kv_capacity, int32_t n_q_heads, int32_t n_kv_heads,
                 int32_t head_dim, float scale, void* workspace, size_t workspace_bytes, hipStream_t stream,
                 bool static_ws = false) {
    if (!q || !k_cache || !v_cache || !o || batch < 1) return KB_ATTN_ERR_INVALID_ARG;
    if (int rc = check_heads(n_q_heads, n_kv_heads, head_dim)) return rc;
    if (int rc = check_scale(scale)) return rc;
    if (n_rows < 1 || n_rows > kDecodeMaxRows) return KB_ATTN_ERR_UNSUPPORTED;
    if (kv_len < n_rows || kv_len > kv_capacity) return KB_ATTN_ERR_LENGTH;
    if (kv_capacity > kMaxLen || batch * n_kv_heads > INT32_MAX) return KB_ATTN_ERR_LENGTH;
    const size_t need = kb_attn_decode_multi_workspace_bytes(batch, n_rows, kv_len, n_q_heads, head_dim);
    if (static_ws) {
        // the scratch array is no caller buffer: nothing can alias it and it
        // is device memory of every device by construction
        if (need > KB_ATTN_DECODE_STATIC_SCRATCH_BYTES) return KB_ATTN_ERR_SCRATCH;
        workspace = nullptr;
        workspace_bytes = 0;
    }
    if (!static_ws && need && (!workspace || workspace_bytes < need)) return KB_ATTN_ERR_WORKSPACE;
    if (int rc = check_aligned({q, k_cache, v_cache, o, need ? workspace : nullptr})) return rc;
    const size_t qbytes = (size_t)batch * n_q_heads * n_rows * kHeadDim * 2;
    const size_t kvbytes = (size_t)batch * n_kv_heads * kv_capacity * kHeadDim * 2;
    if (ranges_overlap(o, qbytes, q, qbytes) || ranges_overlap(o, qbytes, k_cache, kvbytes) ||
        ranges_overlap(o, qbytes, v_cache, kvbytes) || (need && ranges_overlap(o, qbytes, workspace, need)))
        return KB_ATTN_ERR_ALIAS;
    if (need && (ranges_overlap(workspace, need, q, qbytes) || ranges_overlap(workspace, need, k_cache, kvbytes) ||
                 ranges_overlap(workspace, need, v_cache, kvbytes)))
        return KB_ATTN_ERR_ALIAS;
    if (int rc = check_lse(lse, (size_t)batch * n_q_heads * n_rows,
                           {{q, qbytes}, {k_cache, kvbytes}, {v_cache, kvbytes}, {o, qbytes},
                            {need ? workspace : nullptr, need}}))
        return rc;
    if (int rc = check_device({q, k_cache, v_cache, o, need ? workspace : nullptr})) return rc;
    if (static_ws && need)
        if (int rc = static_scratch(&workspace)) return rc;

    const int64_t nc = n_chunks_of(kv_len);
    const int64_t rows = batch * n_q_heads * n_rows;
    DecodeArgs a;
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k_cache;
    a.v = (const uint16_t*)v_cache;
    a.o = (uint16_t*)o;
    a.ws_o = need ? (float*)workspace : nullptr;
    a.ws_ml = need ? (float*)workspace + rows * nc * kHeadDim : nullptr;
    a.lse = lse;
    a.kv_len = kv_len;
    a.cap = kv_capacity;
    a.batch = (int32_t)batch;
    a.n_kv_heads = n_kv_heads;
    a.n_chunks = (int32_t)nc;
    a.n_rows = (int32_t)n_rows;
    a.c = contract_c(scale);
    const int64_t grid = batch * n_kv_heads * nc;
    if (grid > INT32_MAX || rows > INT32_MAX) return KB_ATTN_ERR_LENGTH;
    hipLaunchKernelGGL(decode_kernel, dim3((unsigned)grid), dim3(64 * kDecodeWaves), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return KB_ATTN_ERR_HIP;
    if (nc > 1) {
        CombineArgs cmb;
        cmb.ws_o = a.ws_o;
        cmb.ws_ml = a.ws_ml;
        cmb.o = a.o;
        cmb.lse = lse;
        cmb.kv_len = kv_len;
        cmb.n_chunks = (int32_t)nc;
        cmb.n_rows = (int32_t)n_rows;
        cmb.c = a.c;
        hipLaunchKernelGGL(combine_kernel, dim3((unsigned)rows), dim3(kHeadDim), 0, stream, cmb);
        if (hipGetLastError() != hipSuccess) return KB_ATTN_ERR_HIP;
    }
    return KB_ATTN_OK;
}

}  // namespace

extern "C" {

int kb_attn_prefill(const void* q, const void* k, const void* v, void* o, int64_t batch, int64_t seq_len,
                    int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float scale, hipStream_t stream) {
    return prefill_entry(q, k, v, o, nullptr, batch, seq_len, n_q_heads, n_kv_heads, head_dim, scale, stream);
}

int kb_attn_prefill_lse(const void* q, const void* k, const void* v, void* o, float* lse, int64_t batch,
                        int64_t seq_len, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float scale,
                        hipStream_t stream) {
    if (!lse) return KB_ATTN_ERR_INVALID_ARG;
    return prefill_entry(q, k, v, o, lse, batch, seq_len, n_q_heads, n_kv_heads, head_dim, scale, stream);
}

int kb_attn_partitioned(const void* q, const void* k_cache, const void* v_cache, void* o, int64_t batch,
                        int64_t q_len, int64_t kv_len, int64_t kv_capacity, int32_t n_q_heads, int32_t n_kv_heads,
                        int32_t head_dim, float scale, hipStream_t stream) {
    return partitioned_entry(q, k_cache, v_cache, o, nullptr, batch, q_len, kv_len, kv_capacity, n_q_heads,
                             n_kv_heads, head_dim, scale, stream);
}

int kb_attn_partitioned_lse(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                            int64_t batch, int64_t q_len, int64_t kv_len, int64_t kv_capacity, int32_t n_q_heads,
                            int32_t n_kv_heads, int32_t head_dim, float scale, hipStream_t stream) {
    if (!lse) return KB_ATTN_ERR_INVALID_ARG;
    return partitioned_entry(q, k_cache, v_cache, o, lse, batch, q_len, kv_len, kv_capacity, n_q_heads, n_kv_heads,
                             head_dim, scale, stream);
}

size_t kb_attn_decode_workspace_bytes(int64_t batch, int64_t kv_len, int32_t n_q_heads, int32_t head_dim) {
    if (batch < 1 || kv_len < 1 || n_q_heads < 1 || head_dim != kHeadDim || kv_len > kMaxLen) return 0;
    const int64_t nc = n_chunks_of(kv_len);
    if (nc == 1) return 0;
    return (size_t)batch * n_q_heads * nc * (kHeadDim + 2) * sizeof(float);
}

int kb_attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o, int64_t batch, int64_t kv_len,
                   int64_t kv_capacity, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float scale,
                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return decode_entry(q, k_cache, v_cache, o, nullptr, batch, 1, kv_len, kv_capacity, n_q_heads, n_kv_heads,
                        head_dim, scale, workspace, workspace_bytes, stream);
}

int kb_attn_decode_static(const void* q, const void* k_cache, const void* v_cache, void* o, int64_t batch,
                          int64_t kv_len, int64_t kv_capacity, int32_t n_q_heads, int32_t n_kv_heads,
                          int32_t head_dim, float scale, hipStream_t stream) {
    return decode_entry(q, k_cache, v_cache, o, nullptr, batch, 1, kv_len, kv_capacity, n_q_heads, n_kv_heads,
                        head_dim, scale, nullptr, 0, stream, true);
}

int kb_attn_decode_lse(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int64_t batch,
                       int64_t kv_len, int64_t kv_capacity, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                       float scale, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!lse) return KB_ATTN_ERR_INVALID_ARG;
    return decode_entry(q, k_cache, v_cache, o, lse, batch, 1, kv_len, kv_capacity, n_q_heads, n_kv_heads,
                        head_dim, scale, workspace, workspace_bytes, stream);
}

size_t kb_attn_decode_multi_workspace_bytes(int64_t batch, int64_t n_rows, int64_t kv_len, int32_t n_q_heads,
                                            int32_t head_dim) {
    if (batch < 1 || n_rows < 1 || n_rows > kDecodeMaxRows || kv_len < n_rows || n_q_heads < 1 ||
        head_dim != kHeadDim || kv_len > kMaxLen)
        return 0;
    const int64_t nc = n_chunks_of(kv_len);
    if (nc == 1) return 0;
    return (size_t)batch * n_q_heads * n_rows * nc * (kHeadDim + 2) * sizeof(float);
}

int kb_attn_decode_multi(const void* q, const void* k_cache, const void* v_cache, void* o, int64_t batch,
                         int64_t n_rows, int64_t kv_len, int64_t kv_capacity, int32_t n_q_heads, int32_t n_kv_heads,
                         int32_t head_dim, float scale, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return decode_entry(q, k_cache, v_cache, o, nullptr, batch, n_rows, kv_len, kv_capacity, n_q_heads, n_kv_heads,
                        head_dim, scale, workspace, workspace_bytes, stream);
}

int kb_attn_prefill_varlen(const void* q, const void* k, const void* v, void* o, const int64_t* cu_seqlens,
                           int64_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float scale,
                           hipStream_t stream) {
    if (!q || !k || !v || !o || !cu_seqlens || batch < 1) return KB_ATTN_ERR_INVALID_ARG;
    if (int rc = check_heads(n_q_heads, n_kv_heads, head_dim)) return rc;
    if (int rc = check_scale(scale)) return rc;
    std::vector<RaggedSeq> seqs;
    int64_t q_rows = 0, kv_rows = 0;
    if (int rc = read_ragged(cu_seqlens, cu_seqlens, nullptr, batch, seqs, q_rows, kv_rows)) return rc;
    if (int rc = check_aligned({q, k, v, o})) return rc;
    const size_t qbytes = (size_t)n_q_heads * q_rows * kHeadDim * 2;
    const size_t kvbytes = (size_t)n_kv_heads * kv_rows * kHeadDim * 2;
    if (ranges_overlap(o, qbytes, q, qbytes) || ranges_overlap(o, qbytes, k, kvbytes) ||
        ranges_overlap(o, qbytes, v, kvbytes))
        return KB_ATTN_ERR_ALIAS;
    if (int rc = check_device({q, k, v, o})) return rc;
    return launch_prefill_varlen(q, k, v, o, nullptr, seqs, q_rows, kv_rows, n_kv_heads, scale, stream);
}

int kb_attn_prefill_varlen_lse(const void* q, const void* k, const void* v, void* o, float* lse,
                               const int64_t* cu_seqlens, int64_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                               int32_t head_dim, float scale, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse || !cu_seqlens || batch < 1) return KB_ATTN_ERR_INVALID_ARG;
    if (int rc = check_heads(n_q_heads, n_kv_heads, head_dim)) return rc;
    if (int rc = check_scale(scale)) return rc;
    std::vector<RaggedSeq> seqs;
    int64_t q_rows = 0, kv_rows = 0;
    if (int rc = read_ragged(cu_seqlens, cu_seqlens, nullptr, batch, seqs, q_rows, kv_rows)) return rc;
    if (int rc = check_aligned({q, k, v, o})) return rc;
    const size_t qbytes = (size_t)n_q_heads * q_rows * kHeadDim * 2;
    const size_t kvbytes = (size_t)n_kv_heads * kv_rows * kHeadDim * 2;
    if (ranges_overlap(o, qbytes, q, qbytes) || ranges_overlap(o, qbytes, k, kvbytes) ||
        ranges_overlap(o, qbytes, v, kvbytes))
        return KB_ATTN_ERR_ALIAS;
    if (int rc = check_lse(lse, (size_t)n_q_heads * q_rows, {{q, qbytes}, {k, kvbytes}, {v, kvbytes}, {o, qbytes}}))
        return rc;
    if (int rc = check_device({q, k, v, o})) return rc;
    return launch_prefill_varlen(q, k, v, o, lse, seqs, q_rows, kv_rows, n_kv_heads, scale, stream);
}

int kb_attn_partitioned_varlen(const void* q, const void* k_cache, const void* v_cache, void* o, const int64_t* cu_q,
                               const int64_t* cu_cache, const int64_t* kv_lens, int64_t batch, int32_t n_q_heads,
                               int32_t n_kv_heads, int32_t head_dim, float scale, hipStream_t stream) {
    if (!q || !k_cache || !v_cache || !o || !cu_q || !cu_cache || !kv_lens || batch < 1)
        return KB_ATTN_ERR_INVALID_ARG;
    if (int rc = check_heads(n_q_heads, n_kv_heads, head_dim)) return rc;
    if (int rc = check_scale(scale)) return rc;
    std::vector<RaggedSeq> seqs;
    int64_t q_rows = 0, kv_rows = 0;
    if (int rc = read_ragged(cu_q, cu_cache, kv_lens, batch, seqs, q_rows, kv_rows)) return rc;
    if (int rc = check_aligned({q, k_cache, v_cache, o})) return rc;
    const size_t qbytes = (size_t)n_q_heads * q_rows * kHeadDim * 2;
    const size_t kvbytes = (size_t)n_kv_heads * kv_rows * kHeadDim * 2;
    if (ranges_overlap(o, qbytes, q, qbytes) || ranges_overlap(o, qbytes, k_cache, kvbytes) ||
        ranges_overlap(o, qbytes, v_cache, kvbytes))
        return KB_ATTN_ERR_ALIAS;
    if (int rc = check_device({q, k_cache, v_cache, o})) return rc;
    return launch_prefill_varlen(q, k_cache, v_cache, o, nullptr, seqs, q_rows, kv_rows, n_kv_heads, scale, stream);
}

size_t kb_attn_decode_varlen_workspace_bytes(const int64_t* kv_lens, int64_t batch, int32_t n_q_heads,
                                             int32_t head_dim) {
    if (!kv_lens || batch < 1 || n_q_heads < 1 || head_dim != kHeadDim) return 0;
    int64_t rows = 0;
    for (int64_t i = 0; i < batch; ++i) {
        if (kv_lens[i] < 1 || kv_lens[i] > kMaxLen) return 0;
        const int64_t nc = n_chunks_of(kv_lens[i]);
        if (nc > 1) rows += (int64_t)n_q_heads * nc;
    }
    return (size_t)rows * (kHeadDim + 2) * sizeof(float);
}

int kb_attn_decode_varlen(const void* q, const void* k_cache, const void* v_cache, void* o, const int64_t* cu_cache,
                          const int64_t* kv_lens, int64_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                          int32_t head_dim, float scale, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
    if (!q || !k_cache || !v_cache || !o || !cu_cache || !kv_lens || batch < 1) return KB_ATTN_ERR_INVALID_ARG;
    if (int rc = check_heads(n_q_heads, n_kv_heads, head_dim)) return rc;
    if (int rc = check_scale(scale)) return rc;
    // one query token per sequence: query offsets 0, 1, ..., batch
    std::vector<int64_t> cu_tok((size_t)batch + 1);
    for (int64_t i = 0; i <= batch; ++i) cu_tok[(size_t)i] = i;
    for (int64_t i = 0; i < batch; ++i)
        if (kv_lens[i] < 1) return KB_ATTN_ERR_LENGTH;
    std::vector<RaggedSeq> seqs;
    int64_t q_rows = 0, kv_rows = 0;
    if (int rc = read_ragged(cu_tok.data(), cu_cache, kv_lens, batch, seqs, q_rows, kv_rows)) return rc;
    std::vector<int64_t> ws_row0;
    const int64_t ws_rows = ragged_ws_rows(seqs, n_q_heads, &ws_row0);
    const size_t need = (size_t)ws_rows * (kHeadDim + 2) * sizeof(float);
    if (need && (!workspace || workspace_bytes < need)) return KB_ATTN_ERR_WORKSPACE;
    if (int rc = check_aligned({q, k_cache, v_cache, o, need ? workspace : nullptr})) return rc;
    const size_t qbytes = (size_t)n_q_heads * q_rows * kHeadDim * 2;
    const size_t kvbytes = (size_t)n_kv_heads * kv_rows * kHeadDim * 2;
    if (ranges_overlap(o, qbytes, q, qbytes) || ranges_overlap(o, qbytes, k_cache, kvbytes) ||
        ranges_overlap(o, qbytes, v_cache, kvbytes) || (need && ranges_overlap(o, qbytes, workspace, need)))
        return KB_ATTN_ERR_ALIAS;
    if (need && (ranges_overlap(workspace, need, q, qbytes) || ranges_overlap(workspace, need, k_cache, kvbytes) ||
                 ranges_overlap(workspace, need, v_cache, kvbytes)))
        return KB_ATTN_ERR_ALIAS;
    if (int rc = check_device({q, k_cache, v_cache, o, need ? workspace : nullptr})) return rc;

    DecodeVarlenArgs a;
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k_cache;
    a.v = (const uint16_t*)v_cache;
    a.o = (uint16_t*)o;
    a.ws_o = need ? (float*)workspace : nullptr;
    a.ws_ml = need ? (float*)workspace + ws_rows * kHeadDim : nullptr;
    a.tok_stride = 1;
    a.head_stride = batch;
    a.kv_rows = kv_rows;
    a.block_table = nullptr;
    a.max_pages = 0;
    a.page_size = 0;
    a.n_pages = 0;
    a.n_kv_heads = n_kv_heads;
    a.c = contract_c(scale);
    return launch_decode_tables(a, seqs, ws_row0, n_q_heads, false, stream);
}

int kb_attn_decode_paged(const void* q, const void* k_pages, const void* v_pages, void* o,
                         const int32_t* block_table, int64_t max_pages, const int64_t* kv_lens, int64_t batch,
                         int64_t n_pages, int32_t page_size, int32_t n_q_heads, int32_t n_kv_heads,
                         int32_t head_dim, float scale, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    if (!q || !k_pages || !v_pages || !o || !block_table || !kv_lens || batch < 1 || max_pages < 1 || n_pages < 1)
        return KB_ATTN_ERR_INVALID_ARG;
    if (int rc = check_heads(n_q_heads, n_kv_heads, head_dim)) return rc;
    if (int rc = check_scale(scale)) return rc;
    if (page_size < kTile || page_size % kTile != 0) return KB_ATTN_ERR_UNSUPPORTED;
    if (n_pages > INT32_MAX || max_pages * page_size > kMaxLen || batch > INT32_MAX) return KB_ATTN_ERR_LENGTH;
    std::vector<RaggedSeq> seqs;
    for (int64_t i = 0; i < batch; ++i) {
        if (kv_lens[i] < 1 || kv_lens[i] > max_pages * page_size) return KB_ATTN_ERR_LENGTH;
        seqs.push_back({i, i, 1, 0, kv_lens[i]});
    }
    std::vector<int64_t> ws_row0;
    const int64_t ws_rows = ragged_ws_rows(seqs, n_q_heads, &ws_row0);
    const size_t need = (size_t)ws_rows * (kHeadDim + 2) * sizeof(float);
    if (need && (!workspace || workspace_bytes < need)) return KB_ATTN_ERR_WORKSPACE;
    if (int rc = check_aligned({q, k_pages, v_pages, o, need ? workspace : nullptr})) return rc;
    if ((uintptr_t)block_table & 3u) return KB_ATTN_ERR_ALIGNMENT;
    const size_t qbytes = (size_t)batch * n_q_heads * kHeadDim * 2;
    const size_t poolbytes = (size_t)n_pages * n_kv_heads * page_size * kHeadDim * 2;
    const size_t tbytes = (size_t)batch * max_pages * sizeof(int32_t);
    if (ranges_overlap(o, qbytes, q, qbytes) || ranges_overlap(o, qbytes, k_pages, poolbytes) ||
        ranges_overlap(o, qbytes, v_pages, poolbytes) || ranges_overlap(o, qbytes, block_table, tbytes) ||
        (need && ranges_overlap(o, qbytes, workspace, need)))
        return KB_ATTN_ERR_ALIAS;
    if (need && (ranges_overlap(workspace, need, q, qbytes) || ranges_overlap(workspace, need, k_pages, poolbytes) ||
                 ranges_overlap(workspace, need, v_pages, poolbytes) ||
                 ranges_overlap(workspace, need, block_table, tbytes)))
        return KB_ATTN_ERR_ALIAS;
    if (int rc = check_device({q, k_pages, v_pages, o, block_table, need ? workspace : nullptr})) return rc;

    DecodeVarlenArgs a;
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k_pages;
    a.v = (const uint16_t*)v_pages;
    a.o = (uint16_t*)o;
    a.ws_o = need ? (float*)workspace : nullptr;
    a.ws_ml = need ? (float*)workspace + ws_rows * kHeadDim : nullptr;
    a.tok_stride = n_q_heads;  // q, o [batch, n_q_heads, 128]
    a.head_stride = 1;
    a.kv_rows = 0;
    a.block_table = block_table;
    a.max_pages = max_pages;
    a.page_size = page_size;
    a.n_pages = (int32_t)n_pages;
    a.n_kv_heads = n_kv_heads;
    a.c = contract_c(scale);
    return launch_decode_tables(a, seqs, ws_row0, n_q_heads, true, stream);
}

const char* kb_attn_strerror(int code) {
    switch (code) {
        case KB_ATTN_OK: return "success";
        case KB_ATTN_ERR_INVALID_ARG: return "invalid argument (null pointer, non-positive size or bad scale)";
        case KB_ATTN_ERR_UNSUPPORTED: return "unsupported shape (head_dim must be 128 and n_q_heads 4 * n_kv_heads)";
        case KB_ATTN_ERR_LENGTH: return "bad lengths (need 1 <= q_len <= kv_len <= kv_capacity <= 2^30)";
        case KB_ATTN_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
        case KB_ATTN_ERR_DEVICE: return "pointer is not device memory of the current device";
        case KB_ATTN_ERR_WORKSPACE: return "decode workspace missing or too small";
        case KB_ATTN_ERR_ALIAS: return "output overlaps an input or the workspace";
        case KB_ATTN_ERR_HIP: return "HIP launch failed";
        case KB_ATTN_ERR_SCRATCH: return "the call needs more than the library's 8 MiB static decode scratch";
        default: return "unknown error code";
    }
}

void kb_attn_contract(int32_t* kv_tile, int32_t* kv_chunk, int32_t* version) {
    if (kv_tile) *kv_tile = kTile;
    if (kv_chunk) *kv_chunk = kChunk;
    if (version) *version = KB_ATTN_CONTRACT_VERSION;
}

}  // extern "C"
