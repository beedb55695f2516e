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
//   per row, per tile, in order:
//     s_j   = MFMA chain over d in k-steps 0..7 (step st covers d 16st..16st+15)
//     s_j   = -inf where key j > pos                  (select)
//     mt    = max_j s_j
//     m'    = max(m, mt);  nc = -(m' * c)            with c = fp32(scale * log2 e)
//     a     = (m' == m) ? 1 : exp2(fma(m, c, nc))
//     p_j   = exp2(fma(s_j, c, nc));  P_j = bf16_rne(p_j)
//     l     = fma(l, a, tree_sum(P))                  (fixed tree, see tile_step)
//     o     = o * a;  o = MFMA chain over the tile's 4 key steps in order
//     m     = m'
//   per chunk, in chunk order (first chunk is copied, the rest folded):
//     M' = max(M, m); nc = -(M' c); A = (M' == M) ? 1 : exp2(fma(M, c, nc))
//     B  = (M' == m) ? 1 : exp2(fma(m, c, nc)); L = fma(L, A, l B); O = fma(O, A, o B)
//   out = bf16_rne(O / L)  (IEEE division)
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

// ---------------------------------------------------------------------------
// LDS tile layout (one K/V tile of 64 keys):
//   K   row-major [64 keys][128 d], 256 B per key row, 16-byte chunk c of row
//       r stored at chunk position c ^ (r & 15)  (conflict-free A reads)
//   V^T [128 d][64 keys in MFMA slot order], 128 B per d row, chunk c of row d
//       at chunk position c ^ ((d >> 1) & 7)
// Slot order of V^T: chunk 2*(2*kb+u)+h holds, in order, keys
//   32kb+16u+4h+{0,1,2,3}, 32kb+16u+8+4h+{0,1,2,3}
// which is the key order of the P^T operand taken straight from the S^T
// accumulator (lane half h holds accumulator rows 8b+4h+e).
// ---------------------------------------------------------------------------
constexpr int kKBytes = kTile * kHeadDim * 2;
constexpr int kVBytes = kTile * kHeadDim * 2;
constexpr int kTileBytes = kKBytes + kVBytes;

__device__ __forceinline__ int k_lds_off(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }

__device__ __forceinline__ int vt_lds_off(int d, int chunk) { return d * 128 + ((chunk ^ ((d >> 1) & 7)) << 4); }

// byte offset, inside its V^T row, of key kk (0..63) of the tile
__device__ __forceinline__ int vt_key_chunk(int kk) {
    const int kb = kk >> 5, u = (kk >> 4) & 1, h = (kk >> 2) & 1;
    return 2 * (2 * kb + u) + h;
}
__device__ __forceinline__ int vt_key_byte(int kk) {
    const int a = (kk >> 3) & 1, e = kk & 3;
    return (4 * a + e) * 2;
}

__device__ __forceinline__ bf16x8 lds_read16(const char* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
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
// Staging of one tile from global memory into LDS by a 256-thread workgroup.
// Keys at or beyond kv_len read as zero (never loaded).
// ---------------------------------------------------------------------------
struct Stage {
    u32x4 k[4];
    u32x4 v[2][2];
};

__device__ __forceinline__ void stage_load(Stage& s, const uint16_t* kbase, const uint16_t* vbase,
                                           int64_t key0, int64_t kv_len, int tid) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int u = tid + 256 * i;
        const int row = u >> 4, c = u & 15;
        const int64_t key = key0 + row;
        s.k[i] = key < kv_len ? *reinterpret_cast<const u32x4*>(kbase + key * kHeadDim + c * 8) : zero;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int u = tid + 256 * i;
        const int dg = u >> 5, kp = u & 31;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int64_t key = key0 + 2 * kp + e;
            s.v[i][e] = key < kv_len ? *reinterpret_cast<const u32x4*>(vbase + key * kHeadDim + dg * 8) : zero;
        }
    }
}

__device__ __forceinline__ void stage_store(const Stage& s, char* sK, char* sVt, int tid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int u = tid + 256 * i;
        const int row = u >> 4, c = u & 15;
        *reinterpret_cast<u32x4*>(sK + k_lds_off(row, c)) = s.k[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int u = tid + 256 * i;
        const int dg = u >> 5, kp = u & 31;
        const int kk = 2 * kp;
        const int chunk = vt_key_chunk(kk), byte = vt_key_byte(kk);
#pragma unroll
        for (int d8 = 0; d8 < 8; ++d8) {
            const int word = d8 >> 1, sh = (d8 & 1) * 16;
            const uint32_t lo = (s.v[i][0][word] >> sh) & 0xFFFFu;
            const uint32_t hi = (s.v[i][1][word] >> sh) & 0xFFFFu;
            *reinterpret_cast<uint32_t*>(sVt + vt_lds_off(dg * 8 + d8, chunk) + byte) = lo | (hi << 16);
        }
    }
}

// ---------------------------------------------------------------------------
// One tile of the online softmax for the 32 query columns of a wave.
// Lane l owns query column j = l & 31; lane half h = l >> 5.
//   qf[st]  : B operand of k-step st: Q[query j][16st + 8h .. 16st + 8h + 7]
//   key0    : absolute index of the tile's first key
//   pos     : the column's position (keys > pos are masked) -- used when mask
//   o[db]   : O^T accumulators for d rows 32*(dblk0+db) .. +31 of column j
// ---------------------------------------------------------------------------
template <int NDB>
__device__ __forceinline__ void tile_step(const bf16x8 (&qf)[8], const char* sK, const char* sVt, int lane,
                                          int64_t key0, int64_t pos, bool mask, float c, float& m, float& l,
                                          f32x16 (&o)[NDB], int dblk0) {
    const int j = lane & 31, h = lane >> 5;
    f32x16 s0 = zero16(), s1 = zero16();
#pragma unroll
    for (int st = 0; st < 8; ++st) {
        const bf16x8 k0 = lds_read16(sK + k_lds_off(j, 2 * st + h));
        const bf16x8 k1 = lds_read16(sK + k_lds_off(32 + j, 2 * st + h));
        s0 = mfma(k0, qf[st], s0);
        s1 = mfma(k1, qf[st], s1);
    }
    if (mask) {
        const float ninf = -__builtin_inff();
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t kk = key0 + 8 * (v >> 2) + 4 * h + (v & 3);
            s0[v] = kk > pos ? ninf : s0[v];
            s1[v] = kk + 32 > pos ? ninf : s1[v];
        }
    }
    float mt = s0[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mt = fmaxf(mt, s0[v]);
#pragma unroll
    for (int v = 0; v < 16; ++v) mt = fmaxf(mt, s1[v]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));

    const float mn = fmaxf(m, mt);
    const float nc = -(mn * c);
    const float a = (mn == m) ? 1.0f : exp2_hw(__builtin_fmaf(m, c, nc));

    bf16x8 pf[2][2];
    float w[32];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const __bf16 p0 = (__bf16)exp2_hw(__builtin_fmaf(s0[8 * u + e], c, nc));
            const __bf16 p1 = (__bf16)exp2_hw(__builtin_fmaf(s1[8 * u + e], c, nc));
            pf[0][u][e] = p0;
            pf[1][u][e] = p1;
            w[8 * u + e] = (float)p0;
            w[16 + 8 * u + e] = (float)p1;
        }
    }
    // fixed pairwise tree over the 32 slots (index 16*kb + 8u + e), then the
    // partner lane's half: x + y == y + x, so both halves get the same bits
#pragma unroll
    for (int stride = 1; stride < 32; stride *= 2) {
#pragma unroll
        for (int i = 0; i < 32; i += 2 * stride) w[i] = w[i] + w[i + stride];
    }
    const float ls = w[0] + __shfl_xor(w[0], 32);
    l = __builtin_fmaf(l, a, ls);

#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int v = 0; v < 16; ++v) o[db][v] = o[db][v] * a;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const bf16x8 vf = lds_read16(sVt + vt_lds_off(32 * (dblk0 + db) + j, 2 * (2 * kb + u) + h));
                o[db] = mfma(vf, pf[kb][u], o[db]);
            }
        }
    }
    m = mn;
}

// Fold weights of one chunk into the running total (scalars of one column).
__device__ __forceinline__ void fold_scalars(float M, float m, float c, float& Mn, float& A, float& B) {
    Mn = fmaxf(M, m);
    const float nc = -(Mn * c);
    A = (Mn == M) ? 1.0f : exp2_hw(__builtin_fmaf(M, c, nc));
    B = (Mn == m) ? 1.0f : exp2_hw(__builtin_fmaf(m, c, nc));
}

__device__ __forceinline__ float fold_value(float O, float A, float o, float B) {
    return __builtin_fmaf(O, A, o * B);
}

__device__ __forceinline__ uint16_t finalize(float O, float L) {
    const __bf16 r = (__bf16)(O / L);
    return __builtin_bit_cast(uint16_t, r);
}

}  // namespace kb
