// Gathered block-sparse flash attention and its dense comparator for gfx950.
//
// Method sources (web pages):
//   [hamidun] "AB-Attention speeds up video generation up to 2.23x and skips
//             92% of attention compute", section "three techniques in
//             AB-Attention": SIP paragraph (each chosen block weighted by 1/p,
//             i.e. ordinary softmax attention on shifted logits, one pass) and
//             kernel paragraph (KV blocks of at most 4 tokens gathered by index
//             into full matrix-core tiles, no token reordering, no copies).
//   [edumints] section "three innovations", kernel item (small KV blocks packed
//             into full tensor-core tiles at no extra matrix-core cost).
//
// Design (one workgroup = one plan row = 128 queries of one (b, h); 4 waves,
// wave w owns queries [32w, 32w+32)):
//   * A key tile is 16 KV blocks = 64 keys. The 16 blocks of a tile are the
//     row's next 16 plan entries; each is 4 consecutive tokens, i.e. one
//     contiguous 4*d*2-byte piece of K and of V, so the gather is a set of
//     fully coalesced loads, one per block per wave instruction.
//   * S^T = K Q^T on MFMA 32x32x16 bf16: A = K rows from LDS, B = the wave's
//     Q kept in registers. In the D layout a lane holds one query (column
//     l%32) and 16 keys (rows (i/4)*8 + (l/32)*4 + i%4): the 4 rows i%4 are
//     exactly one KV block, so the block's log-weight is one scalar per group
//     of 4 accumulators, and the row max / sum over keys is lane-local plus
//     one exchange with lane l^32.
//   * O^T = V^T P^T on the same MFMA: B = P taken straight from the S^T
//     accumulators (converted to bf16), A = V^T rows read from a transposed V
//     tile in LDS. The key order inside each 16-key slice follows the
//     accumulator layout (blocks stored in the order 0,2,1,3), so no lane
//     exchange is needed. O^T has the query in the lane's column, so the
//     online-softmax rescale is lane-local.
//   * Tile t+1 is loaded into registers while tile t is computed; one LDS
//     buffer, two barriers per tile, two workgroups per CU.
//   * Workgroup ids are dealt to the 8 XCDs round-robin; rows are assigned so
//     that each XCD takes a contiguous range of rows, keeping neighbouring
//     query blocks of a head (which gather overlapping KV blocks) in one L2.
#include "absa_internal.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace absa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTileBlocks = 16;                 // KV blocks per tile
constexpr int kTileKeys = kTileBlocks * kKvBlock;  // 64
constexpr int kVStride = kTileKeys + 8;         // transposed V row stride (bf16)
constexpr int kXcds = 8;

struct AttnParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    int64_t N, QB, M, rows, per_xcd;
    const int64_t* rowptr;
    const int32_t* idx;
    const float* logw;
    float scale_log2;
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const __bf16 a = static_cast<__bf16>(lo);
    const __bf16 b = static_cast<__bf16>(hi);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// Per-lane prefetch registers for one tile.
template <int D, bool F32> struct TileRegs;
template <int D> struct TileRegs<D, false> {
    uint4 k[D / 32];          // 8 bf16 of one key row
    uint32_t v[D / 32][4];    // channel pair of 4 keys
    float lw[D / 32];
};
template <int D> struct TileRegs<D, true> {
    float4 k[D / 32][2];
    float2 v[D / 32][4];
    float lw[D / 32];
};

template <int D, bool F32, bool DENSE>
__global__ __launch_bounds__(256, 2) void attn_kernel(AttnParams P) {
    constexpr int KS = D + 8;                   // K tile row stride (bf16)
    constexpr int NP = D / 32;                  // loader passes per tile
    constexpr int LPB = D / 2;                  // lanes per KV block in a pass
    constexpr int BPP = 64 / LPB;               // blocks per pass per wave
    constexpr int NS = D / 16;                  // 16-channel MFMA steps
    constexpr int ND = D / 32;                  // 32-channel output blocks
    __shared__ __align__(16) uint16_t Ks[kTileKeys * KS];
    __shared__ __align__(16) uint16_t Vt[D * kVStride];
    __shared__ float lws[kTileBlocks];

    const int bid = blockIdx.x;
    const int64_t row = static_cast<int64_t>(bid % kXcds) * P.per_xcd + bid / kXcds;
    if (row >= P.rows) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int half = lane >> 5;

    const int64_t bh = row / P.QB;
    const int64_t r = row - bh * P.QB;
    const int64_t q0 = r * kQueryBlock;
    const int64_t head_off = bh * P.N * D;

    int64_t base = 0, cnt = P.M;
    if (!DENSE) {
        base = P.rowptr[row];
        cnt = P.rowptr[row + 1] - base;
    }
    const int64_t ntiles = (cnt + kTileBlocks - 1) / kTileBlocks;

    // ---- the wave's queries as the B operand of S^T = K Q^T ----
    const int64_t my_q = q0 + wave * 32 + col;
    const bool wave_active = (q0 + wave * 32) < P.N;
    bf16x8 qb[NS];
    {
        const bool ok = my_q < P.N;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int dd = s * 16 + half * 8;
            uint4 u = make_uint4(0, 0, 0, 0);
            if (ok) {
                if constexpr (F32) {
                    const float* src = static_cast<const float*>(P.q) + head_off + my_q * D + dd;
                    const float4 x0 = *reinterpret_cast<const float4*>(src);
                    const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
                    u = make_uint4(pack_bf16x2(x0.x, x0.y), pack_bf16x2(x0.z, x0.w),
                                   pack_bf16x2(x1.x, x1.y), pack_bf16x2(x1.z, x1.w));
                } else {
                    u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(P.q) +
                                                        head_off + my_q * D + dd);
                }
            }
            qb[s] = as_bf16x8(u);
        }
    }

    // ---- gather of one tile into registers ----
    TileRegs<D, F32> R;
    auto load_tile = [&](int64_t t) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int tb = wave * 4 + p * BPP + lane / LPB;     // block within tile
            const int c = lane % LPB;
            const int64_t gb = t * kTileBlocks + tb;            // block within row
            const bool valid = gb < cnt;
            const int64_t gbc = valid ? gb : (cnt - 1);
            int64_t blk;
            if (DENSE) {
                blk = gbc;
                R.lw[p] = valid ? 0.0f : -INFINITY;
            } else {
                blk = P.idx[base + gbc];
                R.lw[p] = valid ? P.logw[base + gbc] * kLog2e : -INFINITY;
            }
            const int64_t key0 = blk * kKvBlock;
            const int kk = c / (D / 8);
            const int d0 = (c % (D / 8)) * 8;
            if constexpr (F32) {
                const float* ksrc = static_cast<const float*>(P.k) + head_off + (key0 + kk) * D + d0;
                R.k[p][0] = *reinterpret_cast<const float4*>(ksrc);
                R.k[p][1] = *reinterpret_cast<const float4*>(ksrc + 4);
                const float* vsrc = static_cast<const float*>(P.v) + head_off + key0 * D + 2 * c;
#pragma unroll
                for (int t4 = 0; t4 < kKvBlock; ++t4)
                    R.v[p][t4] = *reinterpret_cast<const float2*>(vsrc + t4 * D);
            } else {
                R.k[p] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(P.k) +
                                                         head_off + (key0 + kk) * D + d0);
                const uint32_t* vsrc = reinterpret_cast<const uint32_t*>(
                    static_cast<const uint16_t*>(P.v) + head_off + key0 * D) + c;
#pragma unroll
                for (int t4 = 0; t4 < kKvBlock; ++t4) R.v[p][t4] = vsrc[t4 * (D / 2)];
            }
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int tb = wave * 4 + p * BPP + lane / LPB;
            const int c = lane % LPB;
            const int kk = c / (D / 8);
            const int d0 = (c % (D / 8)) * 8;
            uint4 ku;
            uint32_t v4[4];
            if constexpr (F32) {
                ku = make_uint4(pack_bf16x2(R.k[p][0].x, R.k[p][0].y),
                                pack_bf16x2(R.k[p][0].z, R.k[p][0].w),
                                pack_bf16x2(R.k[p][1].x, R.k[p][1].y),
                                pack_bf16x2(R.k[p][1].z, R.k[p][1].w));
#pragma unroll
                for (int t4 = 0; t4 < 4; ++t4) v4[t4] = pack_bf16x2(R.v[p][t4].x, R.v[p][t4].y);
            } else {
                ku = R.k[p];
#pragma unroll
                for (int t4 = 0; t4 < 4; ++t4) v4[t4] = R.v[p][t4];
            }
            *reinterpret_cast<uint4*>(&Ks[(tb * kKvBlock + kk) * KS + d0]) = ku;
            // V^T: channel 2c gets the low halves of the 4 keys, 2c+1 the high.
            const int grp = tb >> 2, bi = tb & 3;
            const int pcol = grp * 16 + ((bi & 1) * 2 + (bi >> 1)) * 4;   // block order 0,2,1,3
            const uint2 lo = make_uint2((v4[0] & 0xFFFFu) | (v4[1] << 16),
                                        (v4[2] & 0xFFFFu) | (v4[3] << 16));
            const uint2 hi = make_uint2((v4[0] >> 16) | (v4[1] & 0xFFFF0000u),
                                        (v4[2] >> 16) | (v4[3] & 0xFFFF0000u));
            *reinterpret_cast<uint2*>(&Vt[(2 * c) * kVStride + pcol]) = lo;
            *reinterpret_cast<uint2*>(&Vt[(2 * c + 1) * kVStride + pcol]) = hi;
            if (c == 0) lws[tb] = R.lw[p];
        }
    };

    floatx16 O[ND];
#pragma unroll
    for (int j = 0; j < ND; ++j) O[j] = floatx16{};
    float m_run = -INFINITY, l_run = 0.0f;

    if (ntiles > 0) load_tile(0);
    for (int64_t t = 0; t < ntiles; ++t) {
        __syncthreads();
        store_tile();
        __syncthreads();
        if (t + 1 < ntiles) load_tile(t + 1);
        if (!wave_active) continue;

        floatx16 S[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            S[kb] = floatx16{};
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const uint4 a = *reinterpret_cast<const uint4*>(
                    &Ks[(kb * 32 + col) * KS + s * 16 + half * 8]);
                S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qb[s], S[kb], 0, 0, 0);
            }
        }
        // Logits in log2 units with the block log-weight; row max.
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float lw = lws[kb * 8 + 2 * g + half];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = g * 4 + e;
                    S[kb][i] = fmaf(S[kb][i], P.scale_log2, lw);
                    mx = fmaxf(mx, S[kb][i]);
                }
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        const float alpha = exp2f(m_run - m_use);
        m_run = m_new;
        float psum = 0.0f;
        uint4 pb[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                S[kb][i] = exp2f(S[kb][i] - m_use);
                psum += S[kb][i];
            }
#pragma unroll
            for (int sh = 0; sh < 2; ++sh) {
                const int o8 = sh * 8;
                pb[kb * 2 + sh] = make_uint4(pack_bf16x2(S[kb][o8 + 0], S[kb][o8 + 1]),
                                             pack_bf16x2(S[kb][o8 + 2], S[kb][o8 + 3]),
                                             pack_bf16x2(S[kb][o8 + 4], S[kb][o8 + 5]),
                                             pack_bf16x2(S[kb][o8 + 6], S[kb][o8 + 7]));
            }
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int j = 0; j < ND; ++j) {
#pragma unroll
            for (int i = 0; i < 16; ++i) O[j][i] *= alpha;
        }
#pragma unroll
        for (int j = 0; j < ND; ++j) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint4 a = *reinterpret_cast<const uint4*>(
                    &Vt[(j * 32 + col) * kVStride + s * 16 + half * 8]);
                O[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(pb[s]), O[j],
                                                               0, 0, 0);
            }
        }
    }

    if (!wave_active || my_q >= P.N) return;
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = (l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
#pragma unroll
    for (int j = 0; j < ND; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int dd = j * 32 + g * 8 + half * 4;
            const float x0 = O[j][g * 4 + 0] * inv, x1 = O[j][g * 4 + 1] * inv;
            const float x2 = O[j][g * 4 + 2] * inv, x3 = O[j][g * 4 + 3] * inv;
            if constexpr (F32) {
                float* dst = static_cast<float*>(P.o) + head_off + my_q * D + dd;
                *reinterpret_cast<float4*>(dst) = make_float4(x0, x1, x2, x3);
            } else {
                uint16_t* dst = static_cast<uint16_t*>(P.o) + head_off + my_q * D + dd;
                *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
            }
        }
    }
}

template <int D, bool F32, bool DENSE>
void launch_one(const AttnParams& p, hipStream_t s) {
    const int64_t grid = p.per_xcd * kXcds;
    hipLaunchKernelGGL((attn_kernel<D, F32, DENSE>), dim3(static_cast<unsigned>(grid)), dim3(256),
                       0, s, p);
}

}  // namespace

hipError_t launch_attention(const void* q, const void* k, const void* v, void* o, Dtype dt,
                            int64_t B, int64_t H, int64_t N, int d, const int64_t* rowptr,
                            const int32_t* idx, const float* logw, bool dense, hipStream_t s) {
    AttnParams p;
    p.q = q; p.k = k; p.v = v; p.o = o;
    p.N = N;
    p.QB = (N + kQueryBlock - 1) / kQueryBlock;
    p.M = N / kKvBlock;
    p.rows = B * H * p.QB;
    p.per_xcd = (p.rows + kXcds - 1) / kXcds;
    p.rowptr = rowptr; p.idx = idx; p.logw = logw;
    p.scale_log2 = kLog2e / sqrtf(static_cast<float>(d));
    if (p.rows == 0) return hipSuccess;
    const bool f32 = (dt == kF32);
    if (d == 128) {
        if (f32) dense ? launch_one<128, true, true>(p, s) : launch_one<128, true, false>(p, s);
        else dense ? launch_one<128, false, true>(p, s) : launch_one<128, false, false>(p, s);
    } else {
        if (f32) dense ? launch_one<64, true, true>(p, s) : launch_one<64, true, false>(p, s);
        else dense ? launch_one<64, false, true>(p, s) : launch_one<64, false, false>(p, s);
    }
    return hipGetLastError();
}

}  // namespace absa
