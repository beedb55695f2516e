// kb_attn: bitwise-aligned causal GQA attention forward for gfx950 (MI355X).
//
// Three kernels, all built on the contract in kb_contract.h:
//   prefill_kernel  full-sequence prefill and partitioned forward (the same
//                   kernel: row r sits at position kv_len - q_len + r)
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
#include <cstdint>

#include "../../include/kb_attn.h"
#include "kb_contract.h"

namespace kb {

static_assert(KB_ATTN_KV_TILE == kTile && KB_ATTN_KV_CHUNK == kChunk, "header and contract disagree");

struct PrefillArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    int64_t q_len, kv_len, cap;
    int32_t batch, n_kv_heads;
    int32_t pb_first, n_pb;  // 64-position blocks covered by the call
    float c;                 // scale * log2(e), rounded once to fp32
};

constexpr int kPrefillWaves = 8;
constexpr int kStages = 3;

// Workgroup = 8 waves = the 4 query heads of one KV head x 2 halves of the 64
// absolute positions [64 pb, 64 pb + 64).  Every row of the block has its last
// visible key in tile pb, so all rows visit exactly the tiles 0..pb and never
// a tile that is fully masked for them.  K/V tiles are shared by the 8 waves
// through a 3-stage LDS ring filled by direct loads two tiles ahead.
// kPartitioned = false is the full-sequence case (q_len == kv_len, row r at
// position r); both instantiations run the same per-row arithmetic.
template <bool kPartitioned>
__global__ __launch_bounds__(64 * kPrefillWaves) void prefill_kernel(PrefillArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[kStages * kTileBytes];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nbg = a.batch * a.n_kv_heads;
    const int x = blockIdx.x;
    int bg, pbr;
    if ((nbg & 7) == 0) {
        // workgroups are dispatched to the 8 XCDs round-robin (x % 8); give XCD
        // k the (b, g) pairs k, k + 8, ... one after another, each pair's
        // position blocks longest first, so the blocks running together on an
        // XCD stream the same K/V tiles through its L2
        const int i = x >> 3;
        bg = (i / a.n_pb) * 8 + (x & 7);
        pbr = i % a.n_pb;
    } else {
        bg = x % nbg;
        pbr = x / nbg;
    }
    const int pb = a.pb_first + a.n_pb - 1 - pbr;
    const int b = bg / a.n_kv_heads, g = bg % a.n_kv_heads;
    const int n_q_heads = kGroup * a.n_kv_heads;
    const int head = kGroup * g + (w & 3);
    const int j = lane & 31, h = lane >> 5;

    const int64_t off = kPartitioned ? a.kv_len - a.q_len : 0;
    const int64_t pos = (int64_t)pb * 64 + 32 * (w >> 2) + j;
    const int64_t r = pos - off;
    const bool active = r >= 0 && r < a.q_len;

    const int64_t kvoff = ((int64_t)b * a.n_kv_heads + g) * a.cap * kHeadDim;
    const uint16_t* kbase = a.k + kvoff;
    const uint16_t* vbase = a.v + kvoff;
    const int t_last = pb;

    StagePlan<kPrefillWaves> plan;
    stage_plan(plan, lane, w);
    stage_tile(plan, kbase, vbase, 0, a.kv_len, smem, smem + kKBytes, lane, w);
    if (t_last >= 1)
        stage_tile(plan, kbase, vbase, kTile, a.kv_len, smem + kTileBytes, smem + kTileBytes + kKBytes, lane, w);

    bf16x8 qf[8];
    {
        const uint16_t* qrow = a.q + (((int64_t)b * n_q_heads + head) * a.q_len + (active ? r : 0)) * kHeadDim;
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

    // Wait for this wave's loads of tile t, publish it to the workgroup, then
    // start the loads of tile t + 2 into the stage nobody reads any more.
    auto publish = [&](int t) {
        if (t + 1 <= t_last)
            wait_vm<kTileLoads / kPrefillWaves>();
        else
            wait_vm<0>();
        __syncthreads();
        if (t + 2 <= t_last) {
            char* nb = smem + ((t + 2) % kStages) * kTileBytes;
            stage_tile(plan, kbase, vbase, (int64_t)(t + 2) * kTile, a.kv_len, nb, nb + kKBytes, lane, w);
        }
    };
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

    // tiles below the diagonal: every key visible to every row
    for (int t = 0; t < t_last; ++t) {
        publish(t);
        const char* buf = smem + (t % kStages) * kTileBytes;
        tile_step<4, false>(qf, buf, buf + kKBytes, lane, (int64_t)t * kTile, pos, a.c, mc, l, acc, 0);
        if ((t % kTilesPerChunk) == kTilesPerChunk - 1) close_chunk();
    }
    // the diagonal tile t_last holds keys beyond some rows' positions
    {
        publish(t_last);
        const char* buf = smem + (t_last % kStages) * kTileBytes;
        tile_step<4, true>(qf, buf, buf + kKBytes, lane, (int64_t)t_last * kTile, pos, a.c, mc, l, acc, 0);
        close_chunk();
    }

    if (active) {
        uint16_t* orow = a.o + (((int64_t)b * n_q_heads + head) * a.q_len + r) * kHeadDim;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int b4 = 0; b4 < 4; ++b4) {
                const uint32_t e0 = finalize(O[db][4 * b4 + 0], L), e1 = finalize(O[db][4 * b4 + 1], L);
                const uint32_t e2 = finalize(O[db][4 * b4 + 2], L), e3 = finalize(O[db][4 * b4 + 3], L);
                uint2 packed;
                packed.x = e0 | (e1 << 16);
                packed.y = e2 | (e3 << 16);
                *reinterpret_cast<uint2*>(orow + 32 * db + 8 * b4 + 4 * h) = packed;
            }
        }
    }
}

struct DecodeArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* ws_o;   // [batch * n_q_heads * n_chunks][128]
    float* ws_ml;  // [batch * n_q_heads * n_chunks][2]: (max * c, sum)
    int64_t kv_len, cap;
    int32_t batch, n_kv_heads, n_chunks;
    float c;
};

constexpr int kDecodeWaves = 4;
// Two stages (64 KiB of LDS) let two decode workgroups share a CU; measured
// on B=16, L=8192 this streams faster than one workgroup with a deeper ring.
constexpr int kDecodeStages = 2;

// Wait until at most `ahead` tiles of this wave's decode loads are pending.
__device__ __forceinline__ void wait_tiles_decode(int ahead) {
    constexpr int per = kTileLoads / kDecodeWaves;
    switch (ahead) {
        case 0: wait_vm<0>(); break;
        case 1: wait_vm<per>(); break;
        case 2: wait_vm<2 * per>(); break;
        case 3: wait_vm<3 * per>(); break;
        default: wait_vm<4 * per>(); break;
    }
}

// Workgroup = 4 waves on one (batch, KV head, chunk).  The four query heads
// sit in MFMA columns 0..3 (the other columns hold zeros).  Every wave computes
// the scores of the tile; wave w accumulates the output rows d = 32w..32w+31.
// The chunk's tiles stream through a kDecodeStages-deep LDS ring.
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[kDecodeStages * kTileBytes];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int x = blockIdx.x;
    const int chunk = x % a.n_chunks;
    const int bg = x / a.n_chunks;
    const int b = bg / a.n_kv_heads, g = bg % a.n_kv_heads;
    const int n_q_heads = kGroup * a.n_kv_heads;
    const int j = lane & 31, h = lane >> 5;
    const bool active = j < kGroup;
    const int head = kGroup * g + (active ? j : 0);
    const int64_t pos = a.kv_len - 1;

    const int64_t kvoff = ((int64_t)b * a.n_kv_heads + g) * a.cap * kHeadDim;
    const uint16_t* kbase = a.k + kvoff;
    const uint16_t* vbase = a.v + kvoff;
    const int n_tiles = (int)((a.kv_len + kTile - 1) / kTile);
    const int t0 = chunk * kTilesPerChunk;
    const int t1 = min(t0 + kTilesPerChunk, n_tiles);

    // ring of kDecodeStages tiles, loads kDecodeStages - 1 tiles ahead
    StagePlan<kDecodeWaves> plan;
    stage_plan(plan, lane, w);
#pragma unroll
    for (int i = 0; i < kDecodeStages - 1; ++i) {
        if (t0 + i < t1) {
            char* nb = smem + i * kTileBytes;
            stage_tile(plan, kbase, vbase, (int64_t)(t0 + i) * kTile, a.kv_len, nb, nb + kKBytes, lane, w);
        }
    }

    bf16x8 qf[8];
    {
        const uint16_t* qrow = a.q + ((int64_t)b * n_q_heads + head) * kHeadDim;
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const u32x4 x4 = *reinterpret_cast<const u32x4*>(qrow + 16 * st + 8 * h);  // row valid either way
            qf[st] = __builtin_bit_cast(bf16x8, active ? x4 : zero);
        }
    }

    float mc = -__builtin_inff(), l = 0.0f;  // max in log2 units
    f32x16 acc[1];
    acc[0] = zero16();
    for (int t = t0; t < t1; ++t) {
        // tiles issued after tile t and still allowed in flight
        const int ahead = min(t1 - 1, t + kDecodeStages - 2) - t;
        wait_tiles_decode(ahead);
        __syncthreads();
        if (t + kDecodeStages - 1 < t1) {
            char* nb = smem + ((t + kDecodeStages - 1 - t0) % kDecodeStages) * kTileBytes;
            stage_tile(plan, kbase, vbase, (int64_t)(t + kDecodeStages - 1) * kTile, a.kv_len, nb, nb + kKBytes,
                       lane, w);
        }
        const char* buf = smem + ((t - t0) % kDecodeStages) * kTileBytes;
        // only the context's last tile can hold keys beyond kv_len - 1
        if (t < n_tiles - 1)
            tile_step<1, false>(qf, buf, buf + kKBytes, lane, (int64_t)t * kTile, pos, a.c, mc, l, acc, w);
        else
            tile_step<1, true>(qf, buf, buf + kKBytes, lane, (int64_t)t * kTile, pos, a.c, mc, l, acc, w);
    }

    if (!active) return;
    const int64_t row = (int64_t)b * n_q_heads + head;
    if (a.n_chunks == 1) {
        // a single chunk is copied into the total: out = o / l
        uint16_t* orow = a.o + row * kHeadDim;
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
            const uint32_t e0 = finalize(acc[0][4 * b4 + 0], l), e1 = finalize(acc[0][4 * b4 + 1], l);
            const uint32_t e2 = finalize(acc[0][4 * b4 + 2], l), e3 = finalize(acc[0][4 * b4 + 3], l);
            uint2 packed;
            packed.x = e0 | (e1 << 16);
            packed.y = e2 | (e3 << 16);
            *reinterpret_cast<uint2*>(orow + 32 * w + 8 * b4 + 4 * h) = packed;
        }
        return;
    }
    const int64_t prow = row * a.n_chunks + chunk;
    float* po = a.ws_o + prow * kHeadDim;
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
        a.ws_ml[prow * 2 + 0] = mc;
        a.ws_ml[prow * 2 + 1] = l;
    }
}

struct CombineArgs {
    const float* ws_o;
    const float* ws_ml;
    uint16_t* o;
    int32_t n_chunks;
    float c;
};

// One workgroup per (batch, query head), one thread per output element d:
// copy chunk 0, fold chunks 1.. in order, finalize.
__global__ __launch_bounds__(128) void combine_kernel(CombineArgs a) {
    const int64_t row = blockIdx.x;
    const int d = threadIdx.x;
    const int64_t base = row * a.n_chunks;
    float Mc = a.ws_ml[base * 2 + 0];
    float L = a.ws_ml[base * 2 + 1];
    float O = a.ws_o[base * kHeadDim + d];
    for (int k = 1; k < a.n_chunks; ++k) {
        const float mc = a.ws_ml[(base + k) * 2 + 0];
        const float l = a.ws_ml[(base + k) * 2 + 1];
        const float o = a.ws_o[(base + k) * kHeadDim + d];
        float Mcn, A, B;
        fold_scalars(Mc, mc, Mcn, A, B);
        L = __builtin_fmaf(L, A, l * B);
        O = fold_value(O, A, o, B);
        Mc = Mcn;
    }
    a.o[row * kHeadDim + d] = finalize(O, L);
}

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

int launch_prefill(bool partitioned, const void* q, const void* k, const void* v, void* o, int64_t batch,
                   int64_t q_len, int64_t kv_len, int64_t cap, int32_t n_kv_heads, float scale, hipStream_t stream) {
    PrefillArgs a;
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.o = (uint16_t*)o;
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
    if (!partitioned)
        hipLaunchKernelGGL(prefill_kernel<false>, dim3((unsigned)grid), dim3(64 * kPrefillWaves), 0, stream, a);
    else
        hipLaunchKernelGGL(prefill_kernel<true>, dim3((unsigned)grid), dim3(64 * kPrefillWaves), 0, stream, a);
    return hipGetLastError() == hipSuccess ? KB_ATTN_OK : KB_ATTN_ERR_HIP;
}

}  // namespace
}  // namespace kb

using namespace kb;

extern "C" {

int kb_attn_prefill(const void* q, const void* k, const void* v, void* o, int64_t batch, int64_t seq_len,
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
    if (int rc = check_device({q, k, v, o})) return rc;
    return launch_prefill(false, q, k, v, o, batch, seq_len, seq_len, seq_len, n_kv_heads, scale, stream);
}

int kb_attn_partitioned(const void* q, const void* k_cache, const void* v_cache, void* o, int64_t batch,
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
    if (int rc = check_device({q, k_cache, v_cache, o})) return rc;
    return launch_prefill(true, q, k_cache, v_cache, o, batch, q_len, kv_len, kv_capacity, n_kv_heads, scale,
                          stream);
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
    if (!q || !k_cache || !v_cache || !o || batch < 1) return KB_ATTN_ERR_INVALID_ARG;
    if (int rc = check_heads(n_q_heads, n_kv_heads, head_dim)) return rc;
    if (int rc = check_scale(scale)) return rc;
    if (kv_len < 1 || kv_len > kv_capacity) return KB_ATTN_ERR_LENGTH;
    if (kv_capacity > kMaxLen || batch * n_kv_heads > INT32_MAX) return KB_ATTN_ERR_LENGTH;
    const size_t need = kb_attn_decode_workspace_bytes(batch, kv_len, n_q_heads, head_dim);
    if (need && (!workspace || workspace_bytes < need)) return KB_ATTN_ERR_WORKSPACE;
    if (int rc = check_aligned({q, k_cache, v_cache, o, need ? workspace : nullptr})) return rc;
    const size_t qbytes = (size_t)batch * n_q_heads * kHeadDim * 2;
    const size_t kvbytes = (size_t)batch * n_kv_heads * kv_capacity * kHeadDim * 2;
    if (ranges_overlap(o, qbytes, q, qbytes) || ranges_overlap(o, qbytes, k_cache, kvbytes) ||
        ranges_overlap(o, qbytes, v_cache, kvbytes) || (need && ranges_overlap(o, qbytes, workspace, need)))
        return KB_ATTN_ERR_ALIAS;
    if (need && (ranges_overlap(workspace, need, q, qbytes) || ranges_overlap(workspace, need, k_cache, kvbytes) ||
                 ranges_overlap(workspace, need, v_cache, kvbytes)))
        return KB_ATTN_ERR_ALIAS;
    if (int rc = check_device({q, k_cache, v_cache, o, need ? workspace : nullptr})) return rc;

    const int64_t nc = n_chunks_of(kv_len);
    const int64_t rows = batch * n_q_heads;
    DecodeArgs a;
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k_cache;
    a.v = (const uint16_t*)v_cache;
    a.o = (uint16_t*)o;
    a.ws_o = need ? (float*)workspace : nullptr;
    a.ws_ml = need ? (float*)workspace + rows * nc * kHeadDim : nullptr;
    a.kv_len = kv_len;
    a.cap = kv_capacity;
    a.batch = (int32_t)batch;
    a.n_kv_heads = n_kv_heads;
    a.n_chunks = (int32_t)nc;
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
        cmb.n_chunks = (int32_t)nc;
        cmb.c = a.c;
        hipLaunchKernelGGL(combine_kernel, dim3((unsigned)rows), dim3(kHeadDim), 0, stream, cmb);
        if (hipGetLastError() != hipSuccess) return KB_ATTN_ERR_HIP;
    }
    return KB_ATTN_OK;
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
        default: return "unknown error code";
    }
}

void kb_attn_contract(int32_t* kv_tile, int32_t* kv_chunk, int32_t* version) {
    if (kv_tile) *kv_tile = kTile;
    if (kv_chunk) *kv_chunk = kChunk;
    if (version) *version = KB_ATTN_CONTRACT_VERSION;
}

}  // extern "C"
