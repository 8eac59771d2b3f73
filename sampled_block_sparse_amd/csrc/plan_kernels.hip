// Plan kernels for AB-Attention on gfx950: mean keys, IBCS k-means, IBCS
// scores, SIP probabilities / draws / CSR.
//
// Method sources (web pages):
//   [hamidun] "AB-Attention speeds up video generation up to 2.23x and skips
//             92% of attention compute", section "three techniques in
//             AB-Attention", IBCS and SIP paragraphs.
//   [edumints] "AB-Attention: ... Dogru Blok Dikkat Mekanizmasi", section
//             "three innovations".
#include "absa_internal.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace absa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

template <typename T> __device__ __forceinline__ float load_f32(const T* p);
template <> __device__ __forceinline__ float load_f32<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_f32<uint16_t>(const uint16_t* p) {
    return bf16_to_f32(*p);
}

// ---------------------------------------------------------------------------
// Block floating point for the score contraction. A vector x of fp32 values
// with a shared exponent e (every |x_i| < 2^e, e from frexp of the largest
// |x_i|) is represented as integers X_i = rint(x_i 2^(22-e)), |X_i| <= 2^22,
// each split into balanced base-256 digits X = X2 2^16 + X1 2^8 + X0 with
// X1, X0 in [-128, 127] and X2 in [-64, 64], all int8. Rounding to X costs
// at most 2^(e-23) per element.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int bfp_exponent(float amax) {
    int e = 0;
    (void)frexpf(amax, &e);
    return e;
}
__device__ __forceinline__ void bfp_digits(float x, int e, int8_t& d2, int8_t& d1, int8_t& d0) {
    const int X = static_cast<int>(rintf(ldexpf(x, 22 - e)));
    const int x0 = ((X + 128) & 255) - 128;
    const int r = (X - x0) >> 8;
    const int x1 = ((r + 128) & 255) - 128;
    d0 = static_cast<int8_t>(x0);
    d1 = static_cast<int8_t>(x1);
    d2 = static_cast<int8_t>((r - x1) >> 8);
}

// ---------------------------------------------------------------------------
// Mean keys [hamidun, IBCS paragraph: "averaged keys"]:
// kbar[bh, j, :] = (k[bh, 4j] + k[bh, 4j+1] + k[bh, 4j+2] + k[bh, 4j+3]) / 4.
// One thread per (bh, j, 4-channel chunk), a KV block's d/4 threads in
// consecutive lanes; the fp32 sum of four bf16 values is exact unless their
// exponents differ by more than 15. Also writes each mean's block floating
// point form, the operand of the score kernel's matrix products: digit
// planes kq[bh, j, plane, :] (plane 0 = X2) and the exponent kx[bh, j]. The
// fp32 means are written only when kbar is not null (they are exported, not
// used by the scores).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void mean_keys_kernel(const T* __restrict__ k,
                                                        float* __restrict__ kbar,
                                                        int8_t* __restrict__ kq,
                                                        int8_t* __restrict__ kqt,
                                                        int* __restrict__ kx, int64_t chunks,
                                                        int64_t M, int d) {
    const int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const bool ok = c < chunks;
    const int per_row = d >> 2;                 // 16 or 32 lanes per KV block
    const int64_t blk = (ok ? c : chunks - 1) / per_row;            // flattened bh*M + j
    const int d0 = static_cast<int>((ok ? c : chunks - 1) - blk * per_row) << 2;
    const T* src = k + (blk * kKvBlock) * d + d0;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < kKvBlock; ++t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += load_f32(src + t * d + e);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] *= 0.25f;
    // shared exponent of the block's d channels (its lanes are consecutive)
    float amax = fmaxf(fmaxf(fabsf(acc[0]), fabsf(acc[1])), fmaxf(fabsf(acc[2]), fabsf(acc[3])));
    for (int off = 1; off < per_row; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if (!ok) return;
    if (kbar) *reinterpret_cast<float4*>(kbar + blk * d + d0) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    const int ex = bfp_exponent(amax);
    int8_t pl[3][4];
#pragma unroll
    for (int e = 0; e < 4; ++e) bfp_digits(acc[e], ex, pl[0][e], pl[1][e], pl[2][e]);
    uint32_t word[3];
#pragma unroll
    for (int q = 0; q < 3; ++q)
        word[q] = static_cast<uint8_t>(pl[q][0]) | (static_cast<uint32_t>(static_cast<uint8_t>(pl[q][1])) << 8) |
                  (static_cast<uint32_t>(static_cast<uint8_t>(pl[q][2])) << 16) |
                  (static_cast<uint32_t>(static_cast<uint8_t>(pl[q][3])) << 24);
    int8_t* dst = kq + blk * 3 * d + d0;
#pragma unroll
    for (int q = 0; q < 3; ++q) *reinterpret_cast<uint32_t*>(dst + q * d) = word[q];
    if (kqt) {
        // The same digits tile-major, for the fused score kernel's B operands:
        // 16-key tile T, plane q, 64-channel step st form one 1 KB run in
        // MFMA lane order (lane 16 g + j % 16 holds channels 64 st + 16 g ..
        // +16 of key j), so that each operand load reads 1 KB contiguously.
        const int64_t bh = blk / M, j = blk - bh * M;
        const int64_t ntile = (M + 15) / 16;
        const int nstep = d >> 6;
        const int st = d0 >> 6, g = (d0 & 63) >> 4;
        int8_t* tdst = kqt + ((bh * ntile + j / 16) * 3 * nstep + st) * 1024 + g * 256 +
                       (j % 16) * 16 + (d0 & 15);
#pragma unroll
        for (int q = 0; q < 3; ++q) *reinterpret_cast<uint32_t*>(tdst + q * nstep * 1024) = word[q];
    }
    if (d0 == 0) kx[blk] = ex;
}

// Wave sums with DPP row operations: within each 16-lane row by two quad
// permutes and the half-row and row mirrors, then the two row broadcasts
// (rows 1 and 3 take lane 15 of the row before, rows 2 and 3 lane 31);
// lane 63 ends with the total, read into a scalar. (The sums taken here are
// of integers, or of doubles that are multiples of 2^-52 below 2: exact in
// any order.)
template <int CTRL, int ROWS> __device__ __forceinline__ int dpp_move(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS> __device__ __forceinline__ double dpp_move(double v) {
    const int lo = dpp_move<CTRL, ROWS>(__double2loint(v));
    const int hi = dpp_move<CTRL, ROWS>(__double2hiint(v));
    return __hiloint2double(hi, lo);
}
__device__ __forceinline__ int lane63(int v) { return __builtin_amdgcn_readlane(v, 63); }
__device__ __forceinline__ double lane63(double v) {
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), 63),
                            __builtin_amdgcn_readlane(__double2loint(v), 63));
}
// Sum over each 16-lane row, in every lane of the row.
template <typename V> __device__ __forceinline__ V row_sum16(V v) {
    v += dpp_move<0xB1, 0xf>(v);     // quad_perm [1,0,3,2]
    v += dpp_move<0x4E, 0xf>(v);     // quad_perm [2,3,0,1]
    v += dpp_move<0x141, 0xf>(v);    // row_half_mirror
    v += dpp_move<0x140, 0xf>(v);    // row_mirror
    return v;
}
template <typename V> __device__ __forceinline__ V wave_sum(V v) {
    v += dpp_move<0xB1, 0xf>(v);     // quad_perm [1,0,3,2]
    v += dpp_move<0x4E, 0xf>(v);     // quad_perm [2,3,0,1]
    v += dpp_move<0x141, 0xf>(v);    // row_half_mirror
    v += dpp_move<0x140, 0xf>(v);    // row_mirror
    v += dpp_move<0x142, 0xa>(v);    // row_bcast:15 into rows 1 and 3
    v += dpp_move<0x143, 0xc>(v);    // row_bcast:31 into rows 2 and 3
    return lane63(v);
}

// ---------------------------------------------------------------------------
// IBCS k-means [hamidun, IBCS paragraph; edumints, IBCS item]: one workgroup
// per query block. Lloyd iterations in fp64 on the block's queries in their
// original order; initial centroids are the queries floor(m*n/C_eff);
// nearest centroid by squared distance, ties to the smaller index; a cluster
// left empty keeps its centroid. Outputs fp32 centroids [row, C, d] and
// weights [row, C] = member share of the block's n queries under the last
// assignment (C_eff = min(C, n); further clusters are zero with weight 0).
//
// Layout: the queries stay in LDS in their storage type (bf16 or fp32, both
// exact in fp64). The nearest centroid minimises |c_m|^2 - 2 q.c_m (the
// query's own |q|^2 is common to all clusters): thread (i, hd) forms the
// fp64 dot products of query i with every cluster over channel half hd,
// reading the centroids from a [d][NC] fp64 LDS array by broadcast; the two
// halves are added in a fixed order. The rounding differs from summing
// (q - c)^2 only far below the near-tie margins that decide an assignment.
// The update ranks each cluster's members with wave ballots and sums only
// members, so it costs n*d adds. The centroid sums of bf16/fp32 inputs are
// exact in fp64 for any realistic exponent spread, so each centroid is the
// correctly rounded mean whatever the summation order.
// ---------------------------------------------------------------------------
template <typename T> struct QStore;
template <> struct QStore<uint16_t> {
    static constexpr int kPad = 2;            // odd row stride in 32-bit words
    static __device__ __forceinline__ double get(const uint16_t* p) {
        return static_cast<double>(bf16_to_f32(*p));
    }
};
template <> struct QStore<float> {
    static constexpr int kPad = 1;
    static __device__ __forceinline__ double get(const float* p) { return static_cast<double>(*p); }
};

template <typename T, int D, int CH>
__global__ __launch_bounds__(256) void kmeans_kernel(const T* __restrict__ q, int64_t N,
                                                     int64_t QB, int C, int iters,
                                                     float* __restrict__ cent_out,
                                                     float* __restrict__ w_out) {
    constexpr int NC = 2 * CH;                          // cluster slots
    constexpr int QS = D + QStore<T>::kPad;
    constexpr int DH = D / 2;                           // channels per half
    __shared__ __align__(16) T qs[kQueryBlock * QS];
    // centroids, transposed; rows padded to NC + 2 doubles (80 or 144 bytes,
    // still 16-byte aligned for the broadcast reads) so that lanes walking
    // the channels of one cluster spread over the banks
    __shared__ __align__(16) double ct[D][NC + 2];
    __shared__ double part[NC][kQueryBlock];            // dot products over channel half 1
    __shared__ double cc[NC];                           // |c_m|^2
    __shared__ int assign[kQueryBlock], rank_in_wave[kQueryBlock];
    __shared__ int wcnt[2][NC];
    __shared__ int counts[NC], offs[NC];
    __shared__ int members[kQueryBlock];

    const int64_t row = blockIdx.x;
    const int64_t bh = row / QB;
    const int64_t r = row - bh * QB;
    const int64_t lo = r * kQueryBlock;
    const int n = static_cast<int>(min<int64_t>(kQueryBlock, N - lo));
    const int ceff = min(C, n);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const T* qrow = q + (bh * N + lo) * D;

    // 16-byte global loads, stored as four 4-byte words (the padded LDS rows
    // are 4-byte aligned; a row of D values is a whole number of 16 bytes)
    {
        // (all of a thread's loads are issued before its stores, so their
        // latencies overlap; 256 threads, a fixed trip count)
        constexpr int V = 16 / static_cast<int>(sizeof(T));    // values per 16 bytes
        constexpr int PER = kQueryBlock * (D / V) / 256;        // loads per thread
        static_assert(kQueryBlock * (D / V) % 256 == 0, "whole loads per thread");
        const uint4* src = reinterpret_cast<const uint4*>(qrow);
        uint4 u[PER];
#pragma unroll
        for (int r2 = 0; r2 < PER; ++r2) {
            const int e = tid + 256 * r2;
            u[r2] = (e < n * (D / V)) ? src[e] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int r2 = 0; r2 < PER; ++r2) {
            const int e = tid + 256 * r2;
            if (e < n * (D / V)) {
                const int i = e / (D / V), c = (e - i * (D / V)) * V;
                uint32_t* dst = reinterpret_cast<uint32_t*>(qs + i * QS + c);
                dst[0] = u[r2].x;
                dst[1] = u[r2].y;
                dst[2] = u[r2].z;
                dst[3] = u[r2].w;
            }
        }
    }
    __syncthreads();
    for (int e = tid; e < D * NC; e += blockDim.x) {
        const int dd = e / NC, m = e - dd * NC;
        ct[dd][m] = (m < ceff) ? QStore<T>::get(&qs[((m * n) / ceff) * QS + dd]) : 0.0;
    }
    __syncthreads();

    const int i = tid & (kQueryBlock - 1);
    const int hd = tid >> 7;
    for (int it = 0; it < iters; ++it) {
        // |c_m|^2: 16 lanes per cluster slot, a fixed-order lane reduction.
        if (tid < NC * 16) {
            const int m = tid >> 4, sub = tid & 15;
            double a = 0.0;
            for (int dd = sub; dd < D; dd += 16) a = fma(ct[dd][m], ct[dd][m], a);
            a = row_sum16(a);             // the 16 lanes of slot m form one DPP row
            if (sub == 0) cc[m] = a;
        }
        // q_i . c_m over channel half hd, for every cluster slot.
        double dot[NC];
#pragma unroll
        for (int m = 0; m < NC; ++m) dot[m] = 0.0;
        if (i < n) {
            const T* qi = qs + i * QS + hd * DH;
#pragma unroll 4
            for (int dd = 0; dd < DH; ++dd) {
                const double qv = QStore<T>::get(qi + dd);
                const double* cr = &ct[hd * DH + dd][0];
#pragma unroll
                for (int m = 0; m < NC; ++m) dot[m] = fma(qv, cr[m], dot[m]);
            }
            if (hd == 1) {
#pragma unroll
                for (int m = 0; m < NC; ++m) part[m][i] = dot[m];
            }
        }
        __syncthreads();
        // Nearest centroid (ties to the smaller index) and member ranks.
        if (tid < kQueryBlock) {
            int a = -1;
            if (tid < n) {
                double best = 0.0;
#pragma unroll
                for (int m = 0; m < NC; ++m) {
                    const double dist = cc[m] - 2.0 * (dot[m] + part[m][tid]);
                    if (m < ceff && (a < 0 || dist < best)) { best = dist; a = m; }
                }
                assign[tid] = a;
            }
            int rank = 0;
            for (int m = 0; m < ceff; ++m) {
                const uint64_t b = __ballot(a == m);
                if (a == m) rank = __popcll(b & ((1ull << lane) - 1ull));
                if (lane == 0) wcnt[wave][m] = __popcll(b);
            }
            rank_in_wave[tid] = rank;
        }
        __syncthreads();
        if (tid == 0) {
            int o = 0;
            for (int m = 0; m < ceff; ++m) {
                offs[m] = o;
                counts[m] = wcnt[0][m] + wcnt[1][m];
                o += counts[m];
            }
        }
        __syncthreads();
        if (tid < n) {
            const int a = assign[tid];
            const int pos = offs[a] + (tid >= 64 ? wcnt[0][a] : 0) + rank_in_wave[tid];
            members[pos] = tid;
        }
        __syncthreads();
        // Update: each (cluster, channel pair) owned by one thread: one member
        // index read serves both channels (the sums are exact in any order).
        for (int e = tid; e < ceff * (D / 2); e += blockDim.x) {
            const int m = e / (D / 2), dd = (e - m * (D / 2)) * 2;
            const int cnt = counts[m];
            if (cnt) {
                // four independent partial sums per channel
                const int* mem = members + offs[m];
                double sa[4] = {0.0, 0.0, 0.0, 0.0}, sb[4] = {0.0, 0.0, 0.0, 0.0};
                int k = 0;
                for (; k + 4 <= cnt; k += 4) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const T* qp = &qs[mem[k + u] * QS + dd];
                        sa[u] += QStore<T>::get(qp);
                        sb[u] += QStore<T>::get(qp + 1);
                    }
                }
                for (; k < cnt; ++k) {
                    const T* qp = &qs[mem[k] * QS + dd];
                    sa[0] += QStore<T>::get(qp);
                    sb[0] += QStore<T>::get(qp + 1);
                }
                const double nm = static_cast<double>(cnt);
                ct[dd][m] = ((sa[0] + sa[1]) + (sa[2] + sa[3])) / nm;
                ct[dd + 1][m] = ((sb[0] + sb[1]) + (sb[2] + sb[3])) / nm;
            }
        }
        __syncthreads();
    }

    float* co = cent_out + row * C * D;
    for (int e = tid; e < C * D; e += blockDim.x) {
        const int m = e / D, dd = e - m * D;
        co[e] = (m < ceff) ? static_cast<float>(ct[dd][m]) : 0.0f;
    }
    if (tid < C) {
        w_out[row * C + tid] = (tid < ceff)
            ? static_cast<float>(static_cast<double>(counts[tid]) / static_cast<double>(n))
            : 0.0f;
    }
}

// ---------------------------------------------------------------------------
// IBCS scores [hamidun, IBCS paragraph]: for each query block r and KV block
// j, s_j = sum_m w_m * softmax_j(c_m . kbar_j / sqrt(d)), softmax over all M
// KV blocks of the head. This is a dense contraction (centroids x mean keys,
// per head) that must be accurate to 1e-4 relative; it runs on the int8 MFMA
// (32x32x32) on block floating point forms of both operands (three int8
// digits per value, one exponent per mean key and one for a wave's 32
// centroid slots), summing the six digit products of weight >= 2^16 in int32
// accumulators (exact) and combining them in fp32; the result carries about
// 2^-21 of the dot product's scale. A wave owns 32 centroid slots (32/CP
// query blocks of CP slots; slots past C have weight 0) against 64-key tiles
// loaded straight into LDS, as two 32-key subtiles whose products overlap
// the VALU work of the previous subtile. Pass 1 keeps, per centroid row, a
// reference and the sum of the exponentials relative to it, merged across
// lanes; pass 2 recomputes the logits and writes the weighted sum over the
// block's clusters. MFMA D layout (32x32): lane l
// holds column l%32 (a key) and rows (i/4)*8 + (l/32)*4 + i%4 (centroid
// slots) for i < 16; operand layout (int8, K = 32): lane l holds row l%32
// of A and column l%32 of B at k = (l/32)*16 .. +16.
// ---------------------------------------------------------------------------
// Position of 16-byte slot c of key k in the key's row of a score tile
// plane: c ^ score_swizzle(k). Over any 8 (or 16) consecutive keys read at
// the same slot, the addresses fall in distinct 16-byte bank groups of a
// 128-byte (or 256-byte) LDS row, for rows of 128 bytes (D = 128) and of 64
// bytes (D = 64).
template <int D> __device__ __forceinline__ int score_swizzle(int k) {
    return (D == 128) ? ((k & 7) ^ ((k >> 3) & 1)) : (((k >> 1) & 3) ^ ((k >> 3) & 1));
}

// Loads straight from global memory into LDS: lane l's 16 (or 4) bytes from
// base + off land at lds_dst + 16 l (or 4 l); base is wave-uniform, lds_dst
// too (it goes to M0). Written as inline asm so that the compiler does not
// order every later LDS read of the workgroup behind them; lds_load_wait()
// (vmcnt(0)) completes them, and a barrier after it publishes them. The
// s_nop gives the 5 wait states the load needs after a VALU write of its
// base SGPRs (the compiler may restore spilled SGPRs with v_readlane right
// before the asm, and does not check hazards inside it); it also covers
// the one after the M0 write.
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ void lds_load16(const void* base, uint32_t off, void* lds_dst) {
    const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)lds_dst));
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(m0)
                 : "memory");
}
__device__ __forceinline__ void lds_load4(const void* base, uint32_t off, void* lds_dst) {
    const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)lds_dst));
    asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "{m0}"(m0)
                 : "memory");
}
__device__ __forceinline__ void lds_load_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kScoreWaves = 4;
constexpr int kScoreTile = 32;

// Pass 2's exponent bias of centroid m of query block r: the centroid's
// chunk statistics (reference, sum) combined in chunk order into its
// softmax denominator Z (relative to the largest reference R), folded with
// the centroid's weight: w_m 2^(x - R) / Z = 2^(x + log2(w_m / Z) - R).
// -inf for a slot past QB or C, or of weight 0.
__device__ __forceinline__ float score_bias(const float2* __restrict__ part,
                                            const float* __restrict__ w, int64_t bh, int64_t QB,
                                            int C, int nchunks, int64_t r, int m) {
    if (r >= QB || m >= C) return -INFINITY;
    const float2* pp = part + ((bh * QB + r) * C + m) * nchunks;
    float mx = -INFINITY;
    for (int c = 0; c < nchunks; ++c) mx = fmaxf(mx, pp[c].x);
    float z = 0.0f;
    for (int c = 0; c < nchunks; ++c) {
        const float2 q = pp[c];
        if (q.x != -INFINITY) z += q.y * __builtin_amdgcn_exp2f(q.x - mx);
    }
    const float wm = w[(bh * QB + r) * C + m];
    return (wm > 0.0f) ? log2f(wm / z) - mx : -INFINITY;
}

// The bias of every (query block, centroid), computed once between the
// passes: with the keys split into chunks, every pass-2 workgroup would
// otherwise recombine all chunks' statistics for each of its slots.
__global__ __launch_bounds__(256) void score_bias_kernel(const float2* __restrict__ part,
                                                         const float* __restrict__ w, int64_t QB,
                                                         int C, int nchunks, int64_t n,
                                                         float* __restrict__ sbias) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n) return;
    const int64_t rc = i / C;
    const int m = static_cast<int>(i - rc * C);
    const int64_t bh = rc / QB;
    sbias[i] = score_bias(part, w, bh, QB, C, nchunks, rc - bh * QB, m);
}

// The score contraction of one head runs in two passes over key chunks, so
// the grid has (query-block groups) x (heads) x (chunks) workgroups and
// fills the chip whatever the head count. Pass 1 (PASS2 = false) writes, per centroid and chunk, the running
// max and sum of the centroid's exponentials over the chunk's keys; pass 2
// combines a centroid's chunk statistics in chunk order (deterministic),
// then recomputes the chunk's logits and writes the weighted sums.
template <int CP, int D, bool PASS2>
__global__ __launch_bounds__(256, 2) void scores_kernel(const float* __restrict__ cent,
                                                        const float* __restrict__ w,
                                                        const int8_t* __restrict__ kq,
                                                        const int* __restrict__ kx,
                                                        int64_t QB, int64_t M, int C,
                                                        int chunk_tiles, int nchunks,
                                                        float scale_log2,
                                                        float2* __restrict__ part,
                                                        const float* __restrict__ sbias,
                                                        float* __restrict__ scores) {
    constexpr int RPW = 32 / CP;                    // query blocks per wave
    constexpr int NSTEP = D / 32;                   // MFMA k-steps (32 channels each)
    constexpr int TK = 2 * kScoreTile;              // keys per LDS tile (two 32-key subtiles)
    constexpr int PL = TK * D;                      // bytes of one digit plane of a tile
    constexpr int SPR = D / 16;                     // 16-byte slots per key row of a plane
    constexpr int SLOTS = 3 * TK * SPR;             // slots per LDS tile: a multiple of 256
    static_assert(SLOTS % 256 == 0, "tile slots must split evenly over the threads");
    __shared__ __align__(16) int8_t ks[2][3 * PL];
    __shared__ int kxs[2][TK];                      // exponents of the tile's mean keys

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int half = lane >> 5;
    const int64_t bh = blockIdx.y;
    const int64_t r0 = (static_cast<int64_t>(blockIdx.x) * kScoreWaves + wave) * RPW;
    const int chunk = blockIdx.z;
    const int64_t ntiles = (M + kScoreTile - 1) / kScoreTile;
    const int64_t t0 = static_cast<int64_t>(chunk) * chunk_tiles;
    const int64_t t1 = (t0 + chunk_tiles < ntiles) ? t0 + chunk_tiles : ntiles;

    // A operands: this lane's centroid slot (row col of the 32x32 block),
    // channels s*32 + half*16 .. +16 of each step, as the three int8 digit
    // planes of the centroid's block floating point form.
    const int64_t my_r = r0 + col / CP;
    const int my_m = col % CP;
    const bool slot_ok = (my_r < QB) && (my_m < C);
    typedef int intx4 __attribute__((ext_vector_type(4)));
    intx4 a2[NSTEP], a1[NSTEP], a0[NSTEP];
    float rowf;
    {
        const float* src = cent + ((bh * QB + my_r) * C + my_m) * D;
        float amax = 0.0f;
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                amax = fmaxf(amax, slot_ok ? fabsf(src[st * 32 + half * 16 + e]) : 0.0f);
        }
        // one exponent for the wave's 32 slots (query blocks r0 .. r0 + 32/CP):
        // the row factor is then one scalar, folded into each key's factor
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
        const int ex = bfp_exponent(amax);
        // the log2-domain scale times 2^(e_c - 28): the digit sums carry
        // 2^(44 - e_c - e_k), and the combination below 2^-16
        rowf = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(ldexpf(scale_log2, ex - 28))));
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
            int8_t h2[16], h1[16], h0[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float x = slot_ok ? src[st * 32 + half * 16 + e] : 0.0f;
                bfp_digits(x, ex, h2[e], h1[e], h0[e]);
            }
            __builtin_memcpy(&a2[st], h2, 16);
            __builtin_memcpy(&a1[st], h1, 16);
            __builtin_memcpy(&a0[st], h0, 16);
        }
    }
    __syncthreads();

    // Accumulator row i of this lane is centroid slot (i/4)*8 + half*4 + i%4.
    auto slot_of = [&](int i) { return (i >> 2) * 8 + half * 4 + (i & 3); };
    auto slot_valid = [&](int slot) {
        return (r0 + slot / CP < QB) && (slot % CP < C);
    };
    auto part_index = [&](int slot) {
        return ((bh * QB + r0 + slot / CP) * C + slot % CP) * nchunks;
    };

    const int8_t* kb = kq + bh * M * 3 * D;
    const int* kxb = kx + bh * M;
    const int64_t nsub = t1 - t0;                   // 32-key subtiles of this chunk
    const int64_t nlt = (nsub + 1) / 2;             // 64-key LDS tiles
    if (nsub <= 0) return;                          // (no empty chunk is launched)
    // LDS tile u holds keys (t0 + 2u) * 32 .. +64 plane by plane (X2, X1, X0;
    // a key's row of a plane is D bytes), loaded straight into LDS: the
    // waves' 64-lane loads fill consecutive 1 KB runs of slots. Slot c of key
    // k is stored at c ^ score_swizzle(k) within the row, so that the B
    // operand reads (one slot of 32 consecutive keys) hit distinct banks; a
    // stored slot's key and logical slot follow from its position. Keys past
    // M repeat key M-1 (their logits are never used).
    // A lane's offset within a tile does not depend on the tile, so a tile
    // whose 64 keys all lie below M adds its start to the loads' scalar base
    // (scalar arithmetic) and reuses the lane offsets computed once here.
    // The last tile of a ragged row clamps its keys per lane instead, with
    // 32-bit index arithmetic (M < 2^19) recomputed there; the opaque copy of
    // the lane index keeps the compiler from hoisting that path's per-lane
    // offsets out of the loop.
    const int M32 = static_cast<int>(M);
    uint32_t goff[SLOTS / 256];
    {
        const int lk = lane / SPR, cs = lane % SPR;
#pragma unroll
        for (int i = 0; i < SLOTS / 256; ++i) {
            const int sw = i * 256 + wave * 64;
            const int k = (sw / SPR) % TK + lk;
            goff[i] = static_cast<uint32_t>(k * (3 * D) + (sw / (TK * SPR)) * D +
                                            (cs ^ score_swizzle<D>(k)) * 16);
            asm volatile("" : "+v"(goff[i]));
        }
    }
    auto dma_tile = [&](int buf, int64_t u) __attribute__((always_inline)) {
        const int j0 = static_cast<int>((t0 + 2 * u) * kScoreTile);
        if (j0 + TK <= M32) {
            const int8_t* tb = kb + static_cast<int64_t>(j0) * (3 * D);
#pragma unroll
            for (int i = 0; i < SLOTS / 256; ++i)
                lds_load16(tb, goff[i], &ks[buf][(i * 256 + wave * 64) * 16]);
            if (wave == 0) lds_load4(kxb + j0, static_cast<uint32_t>(lane * 4), &kxs[buf][0]);
            return;
        }
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int lk = ln / SPR, cs = ln % SPR;    // key offset and stored slot of the lane
#pragma unroll
        for (int i = 0; i < SLOTS / 256; ++i) {
            const int sw = i * 256 + wave * 64;     // wave-uniform; a run stays in one plane
            const int p = sw / (TK * SPR);
            const int k = (sw / SPR) % TK + lk;
            const int c = cs ^ score_swizzle<D>(k);
            const int j = min(j0 + k, M32 - 1);
            // j < 2^19: a full-rate 24-bit multiply
            const uint32_t off = __umul24(static_cast<uint32_t>(j), 3 * D) + p * D + c * 16;
            lds_load16(kb, off, &ks[buf][sw * 16]);
        }
        if (wave == 0) {
            const int j = min(j0 + ln, M32 - 1);
            lds_load4(kxb, static_cast<uint32_t>(j * 4), &kxs[buf][0]);
        }
    };
    typedef int intx16 __attribute__((ext_vector_type(16)));
    // Logit of accumulator row k, up to the key's factor: the six digit
    // products of weight >= 2^16 (X2Y2; X2Y1 + X1Y2; X2Y0 + X1Y1 + X0Y2)
    // combined as 2^16 P22 + (2^8 P21 + P20) (the bracket is exact in int32:
    // |P21| <= 2^21, |P20| < 2^23). The logit is this times key_factor (the
    // row factor times 2^(key exponent)); the dropped products are below
    // 2^-21 of the largest |c| |k| of the wave's centroids.
    auto combine = [&](const intx16& i22, const intx16& i21, const intx16& i20,
                       int k) __attribute__((always_inline)) {
        const int lo = (i21[k] << 8) + i20[k];
        return fmaf(static_cast<float>(i22[k]), 65536.0f, static_cast<float>(lo));
    };
    // row factor times 2^(key exponent): the logit is combine(...) times this
    auto key_factor = [&](int buf, int key) __attribute__((always_inline)) {
        return ldexpf(rowf, kxs[buf][key]);
    };
    // One subtile's digit products (subtile sb of buffer buf) into o22/o21/o20,
    // with item(k) (the VALU work of row k of the previous subtile) spread
    // between the MFMAs; the B operands are read one k-step ahead.
    constexpr int NM = 6 * NSTEP;
    auto phase = [&](int buf, int sb, intx16& o22, intx16& o21, intx16& o20,
                     auto&& item) __attribute__((always_inline)) {
        const int key = sb * kScoreTile + col;
        const int8_t* kr = &ks[buf][key * D];
        const int sz = score_swizzle<D>(key);
        // plane p, k-step st: logical slot 2 st + half of the key's row
        auto ld = [&](int p, int st) {
            return *reinterpret_cast<const intx4*>(kr + p * PL + 16 * ((2 * st + half) ^ sz));
        };
        intx4 b2 = ld(0, 0), b1 = ld(1, 0), b0 = ld(2, 0);
        o22 = intx16{};
        o21 = intx16{};
        o20 = intx16{};
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
            intx4 n2 = b2, n1 = b1, n0 = b0;
            if (st + 1 < NSTEP) {
                n2 = ld(0, st + 1);
                n1 = ld(1, st + 1);
                n0 = ld(2, st + 1);
            }
#pragma unroll
            for (int m = 0; m < 6; ++m) {
                if (m == 0) o20 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a2[st], b0, o20, 0, 0, 0);
                if (m == 1) o21 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a2[st], b1, o21, 0, 0, 0);
                if (m == 2) o22 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a2[st], b2, o22, 0, 0, 0);
                if (m == 3) o20 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1[st], b1, o20, 0, 0, 0);
                if (m == 4) o21 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1[st], b2, o21, 0, 0, 0);
                if (m == 5) o20 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0[st], b2, o20, 0, 0, 0);
                const int mi = st * 6 + m;
#pragma unroll
                for (int k = mi * 16 / NM; k < (mi + 1) * 16 / NM; ++k) item(k);
                __builtin_amdgcn_sched_barrier(0);
            }
            b2 = n2;
            b1 = n1;
            b0 = n0;
        }
    };
    // Pipeline over LDS tiles, one barrier per tile: iteration u runs the
    // products of subtile 2u+1 (into set B) beside the VALU work of subtile
    // 2u (set A), then, after the barrier that publishes tile u+1 (loaded
    // from the start of iteration u into the other buffer, which iteration
    // u-1 finished reading before its barrier), the products of subtile
    // 2u+2 (set A) beside the VALU work of subtile 2u+1 (set B). item(...)
    // does the VALU work of one row of a subtile given its accumulators and
    // key factor, post(g, ...) finishes subtile g after its phase, and
    // first(...) runs on subtile 0 alone before the loop.
    intx16 xa22, xa21, xa20, xb22, xb21, xb20;
    auto pipeline = [&](auto&& item, auto&& pre, auto&& post, auto&& first,
                        auto&& after_barrier) __attribute__((always_inline)) {
        auto none = [](int) {};
        dma_tile(0, 0);
        lds_load_wait();
        __syncthreads();
        phase(0, 0, xa22, xa21, xa20, none);
        first(xa22, xa21, xa20, key_factor(0, col));
        for (int64_t u = 0; u < nlt; ++u) {
            const int buf = static_cast<int>(u & 1);
            if (u + 1 < nlt) dma_tile(buf ^ 1, u + 1);
            {
                const float cf = key_factor(buf, col);
                pre();
                phase(buf, 1, xb22, xb21, xb20,
                      [&](int k) { item(xa22, xa21, xa20, cf, k); });
                post(2 * u, xa22, xa21, xa20, cf);
            }
            // key factor of subtile 2u+1, read before the barrier after which
            // the next iteration's loads may overwrite this buffer
            const float cf1 = key_factor(buf, kScoreTile + col);
            lds_load_wait();
            __syncthreads();
            after_barrier();
            if (2 * u + 1 < nsub) {
                pre();
                phase(buf ^ 1, 0, xa22, xa21, xa20,
                      [&](int k) { item(xb22, xb21, xb20, cf1, k); });
                post(2 * u + 1, xb22, xb21, xb20, cf1);
            }
        }
    };
    // A lane's key lies past M only in the last subtile of the row.
    const bool ragged = (M % kScoreTile) != 0;

    if constexpr (!PASS2) {
        // Per centroid row: a reference R (the row's largest logit seen at
        // the last re-basing, the same in all 32 lanes of the half holding
        // the row) and the sum of exp2(x - R - kSlack) over this lane's
        // keys. Kept as nref = -(R + kSlack). A subtile whose logits all stay
        // within R + kSlack costs one FMA, one exponential and one add per
        // logit (computed beside the next subtile's products); otherwise
        // (and on the first and the ragged subtile) the rows are re-based on
        // their new maxima, a wave-uniform branch.
        constexpr float kSlack = 16.0f;
        float nref[16], zs[16], dv[16];
        // Re-basing of row i on the logits x of a subtile (x = -inf past M):
        // R = max(R, the half's largest x), the sum rescaled to the new R.
        auto rebase = [&](int i, float x) __attribute__((always_inline)) {
            float m = x;
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
            const float r_old = -nref[i] - kSlack;
            if (m > r_old) {
                // r_old = -inf only on subtile 0, where zs = 0
                zs[i] = (r_old == -INFINITY) ? 0.0f : zs[i] * __builtin_amdgcn_exp2f(r_old - m);
                nref[i] = -(m + kSlack);
            }
        };
#pragma unroll
        for (int i = 0; i < 16; ++i) { nref[i] = INFINITY; zs[i] = 0.0f; }
        // Subtile 0 sets the references from its exact logits.
        auto first = [&](const intx16& i22, const intx16& i21, const intx16& i20,
                         float cf) __attribute__((always_inline)) {
            const bool ok = t0 * kScoreTile + col < M;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float x = ok ? combine(i22, i21, i20, i) * cf : -INFINITY;
                rebase(i, x);
                zs[i] += __builtin_amdgcn_exp2f(x + nref[i]);
            }
        };
        auto item = [&](const intx16& i22, const intx16& i21, const intx16& i20,
                        float cf, int k) __attribute__((always_inline)) {
            dv[k] = fmaf(combine(i22, i21, i20, k), cf, nref[k]);
            // pinned here, between the MFMAs: the compiler would otherwise
            // sink the whole computation past them, next to its use
            asm volatile("" : "+v"(dv[k]));
        };
        auto pre = [&]() __attribute__((always_inline)) {};
        // Subtiles g >= 1 (the references are finite, so x = dv - nref): a
        // rare re-basing rewrites dv in place, then every subtile adds its
        // exponentials.
        auto post = [&](int64_t g, const intx16&, const intx16&, const intx16&,
                        float) __attribute__((always_inline)) {
            if (g == 0) return;
            const int64_t t = t0 + g;
            const bool last_ragged = ragged && (t + 1) * kScoreTile > M;
            // some dv > 0: the largest bit pattern read as a signed integer is
            // positive (integer maxima: no NaN quieting of the operands)
            int mb = __float_as_int(dv[0]);
#pragma unroll
            for (int i = 1; i < 16; ++i) mb = max(mb, __float_as_int(dv[i]));
            const bool over = mb > 0;
            if (last_ragged || __builtin_amdgcn_ballot_w64(over) != 0) {
                const bool ok = t * kScoreTile + col < M;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float x = ok ? dv[i] - nref[i] : -INFINITY;
                    rebase(i, x);
                    dv[i] = x + nref[i];
                }
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) zs[i] += __builtin_amdgcn_exp2f(dv[i]);
        };
        pipeline(item, pre, post, first, [] {});
        // The reference is uniform over each half: the sums add across its
        // 32 lanes (xor over lane bits 0..4). Chunk statistic of a row:
        // (R + kSlack, sum), i.e. the chunk's sum of 2^x is sum * 2^(R + kSlack).
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) {
#pragma unroll
            for (int i = 0; i < 16; ++i) zs[i] += __shfl_xor(zs[i], off);
        }
        if (col == 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int slot = slot_of(i);
                if (slot_valid(slot)) part[part_index(slot) + chunk] = make_float2(-nref[i], zs[i]);
            }
        }
    } else {
        // Each centroid's exponent bias (score_bias, computed once per
        // centroid by score_bias_kernel): w_m * 2^(x - R) / Z =
        // 2^(x + log2(w_m / Z) - R); -inf for unused slots (weight 0).
        float bias[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int slot = slot_of(i);
            bias[i] = slot_valid(slot) ? sbias[(bh * QB + r0 + slot / CP) * C + slot % CP]
                                       : -INFINITY;
        }
        float pr[RPW];
        auto item = [&](const intx16& i22, const intx16& i21, const intx16& i20,
                        float cf, int k) __attribute__((always_inline)) {
            const float e = __builtin_amdgcn_exp2f(fmaf(combine(i22, i21, i20, k), cf, bias[k]));
            if constexpr (CP == 2) {
                // row (k/4)*4 + 2*half + (k%4)/2: both candidates updated with
                // compile-time indices (indexing by the lane's half spills)
                const int q0 = (k >> 2) * 4 + ((k & 3) >> 1);
                pr[q0] += half ? 0.0f : e;
                pr[q0 + 2] += half ? e : 0.0f;
            } else {
                pr[slot_of(k) / CP] += e;
            }
        };
        auto pre = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int g = 0; g < RPW; ++g) pr[g] = 0.0f;
        };
        // The scores of a subtile are written after the next barrier when the
        // subtile is the first of its LDS tile: written at once, their stores
        // would sit behind the tile loads issued earlier in the iteration and
        // the barrier's wait for those loads would wait for them too. (Not
        // with 16 or 32 rows per wave, C <= 2: the held values would spill.)
        constexpr bool kDefer = RPW <= 8;
        float held[kDefer ? RPW : 1];
        int64_t held_g = -1;
        auto store = [&](int64_t g, const float (&vals)[RPW]) __attribute__((always_inline)) {
            const int jt = static_cast<int>((t0 + g) * kScoreTile);        // < M < 2^19
            const bool ok = jt + col < M32;
#pragma unroll
            for (int q = 0; q < RPW; ++q) {
                // rows q whose slots lie in this lane's half
                const int half_of_q = (CP >= 8) ? (q & 1) : (((q * CP) >> 2) & 1);
                const int64_t rr = r0 + q;
                if (half_of_q == half && rr < QB && ok) {
                    // a wave-uniform row pointer: the lane adds only its column
                    float* rowp = scores + (bh * QB + rr) * M + jt;
                    rowp[col] = vals[q];
                }
            }
        };
        auto post = [&](int64_t g, const intx16&, const intx16&, const intx16&,
                        float) __attribute__((always_inline)) {
            if constexpr (!kDefer) {
                // 16 or 32 rows per wave: written at once, 64-bit addresses per
                // lane (wave-uniform row pointers for every row would stay live
                // across the loop and spill)
                const int64_t j = (t0 + g) * kScoreTile + col;
#pragma unroll
                for (int q = 0; q < RPW; ++q) {
                    const int half_of_q = ((q * CP) >> 2) & 1;
                    const int64_t rr = r0 + q;
                    if (half_of_q == half && rr < QB && j < M) scores[(bh * QB + rr) * M + j] = pr[q];
                }
                return;
            }
            float vals[RPW];
#pragma unroll
            for (int q = 0; q < RPW; ++q) {
                // CP >= 8: a query block's clusters span both halves: add the
                // partner's (one lane exchange)
                if (CP >= 8) {
                    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(pr[q]),
                                                                    __float_as_int(pr[q]), false, false);
                    vals[q] = __int_as_float(r[0]) + __int_as_float(r[1]);
                } else {
                    vals[q] = pr[q];
                }
            }
            if constexpr (kDefer) {
                if ((g & 1) == 0) {
#pragma unroll
                    for (int q = 0; q < RPW; ++q) held[q] = vals[q];
                    held_g = g;
                    return;
                }
            }
            store(g, vals);
        };
        auto after_barrier = [&]() __attribute__((always_inline)) {
            if constexpr (kDefer) {
                if (held_g >= 0) {
                    store(held_g, held);
                    held_g = -1;
                }
            }
        };
        pipeline(item, pre, post, [](const intx16&, const intx16&, const intx16&, float) {},
                 after_barrier);
    }
}

// ---------------------------------------------------------------------------
// Block-wide reductions.
// ---------------------------------------------------------------------------
template <typename V> __device__ V block_sum(V v, V* red) {
    v = wave_sum(v);
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    V t = 0;
    for (int k = 0; k < static_cast<int>(blockDim.x >> 6); ++k) t += red[k];
    return t;
}

// An int and a double summed over the block with one barrier: the caller
// alternates between two sets of slots (redi/redd and redi + 16/redd + 16),
// so a slot is written again only after a later barrier that every wave
// reaches after reading it.
__device__ void block_sum2(int a, double b, int* redi, double* redd, int& ta, double& tb) {
    a = wave_sum(a);
    b = wave_sum(b);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        redi[wave] = a;
        redd[wave] = b;
    }
    __syncthreads();
    ta = 0;
    tb = 0.0;
    for (int k = 0; k < static_cast<int>(blockDim.x >> 6); ++k) {
        ta += redi[k];
        tb += redd[k];
    }
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): 4-word counter, 2-word
// key; 10 rounds of two 32x32->64 multiplies with the Weyl key schedule.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void philox_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
    constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
    for (int rnd = 0; rnd < 10; ++rnd) {
        const uint64_t p0 = static_cast<uint64_t>(M0) * c[0];
        const uint64_t p1 = static_cast<uint64_t>(M1) * c[2];
        const uint32_t hi0 = static_cast<uint32_t>(p0 >> 32), lo0 = static_cast<uint32_t>(p0);
        const uint32_t hi1 = static_cast<uint32_t>(p1 >> 32), lo1 = static_cast<uint32_t>(p1);
        const uint32_t n0 = hi1 ^ c[1] ^ k0;
        const uint32_t n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
        k0 += W0; k1 += W1;
    }
}

// Uniforms in [0, 1) for KV blocks 2i and 2i+1 of row (b, h, r): one
// Philox call with counter (i, r, h, b); block 2i takes the 53 high bits of
// output words 0 and 1, block 2i+1 those of words 2 and 3.
__device__ __forceinline__ void sip_uniform_pair(uint64_t seed, int64_t b, int64_t h, int64_t r,
                                                 int64_t i, double& u0, double& u1) {
    uint32_t c[4] = {static_cast<uint32_t>(i), static_cast<uint32_t>(r),
                     static_cast<uint32_t>(h), static_cast<uint32_t>(b)};
    philox_10(c, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
    u0 = static_cast<double>(((static_cast<uint64_t>(c[0]) << 32) | c[1]) >> 11) * 0x1.0p-53;
    u1 = static_cast<double>(((static_cast<uint64_t>(c[2]) << 32) | c[3]) >> 11) * 0x1.0p-53;
}

// Fixed-size design: the row's uniform U in [0, 2^40), from the Philox
// counter (2^32 - 1, r, h, b) (block pairs never reach that index), words
// (x0, x1) as (hi, lo).
__device__ __forceinline__ uint64_t sys_uniform(uint64_t seed, int64_t b, int64_t h, int64_t r) {
    uint32_t c[4] = {0xFFFFFFFFu, static_cast<uint32_t>(r), static_cast<uint32_t>(h),
                     static_cast<uint32_t>(b)};
    philox_10(c, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
    return ((static_cast<uint64_t>(c[0]) << 32) | c[1]) >> 24;
}
// P = floor(p 2^40) for p in [0, 1]: exact (a power-of-two scaling, then floor)
__device__ __forceinline__ uint64_t sys_size(double p) {
    return static_cast<uint64_t>(floor(p * 0x1.0p40));
}
// number of points U + k 2^40 (k >= 0) below x
__device__ __forceinline__ uint64_t sys_points_below(uint64_t x, uint64_t U) {
    return x > U ? ((x - U - 1) >> 40) + 1 : 0;
}
// 64-bit sum over the wave, the inclusive scan over its lanes, and the scan's
// last value (the wave total), in fixed orders (integers: exact anyway)
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}
__device__ __forceinline__ uint64_t wave_scan_u64(uint64_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint64_t t = __shfl_up(v, off);
        if (lane >= off) v += t;
    }
    return v;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), lane);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), lane);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_last_u64(uint64_t v) { return readlane_u64(v, 63); }

// floor(s * 2^52) of an fp32 score in [0, 1], as an exact fp64 integer. Sums
// of such integers below 2^53 are exact in fp64 in any order, which is the
// order-free fixed-point arithmetic the sampler's rule asks for.
__device__ __forceinline__ double fixed_point(float s) {
    return floor(static_cast<double>(s) * 0x1.0p52);
}

// Sum of fixed-point scores kept in two parts: scores >= 2^-29 have an ulp of
// at least 2^-52, so floor(s * 2^52) = s * 2^52 exactly and they are summed as
// s (every such sum is a multiple of 2^-52 below 2: exact); smaller scores are
// summed as fixed_point(s). value() = 2^52 * big + small, both exact integers
// below 2^53, so the sum is the same exact integer in any order.
struct FixedSum {
    double big = 0.0, small = 0.0;
    __device__ __forceinline__ void add(float s) {
        if (s >= 0x1.0p-29f) big += static_cast<double>(s);
        else small += fixed_point(s);
    }
    __device__ __forceinline__ double value() const { return big * 0x1.0p52 + small; }
};

// p of block j given the row's outcome; capped blocks have p = 1.
__device__ __forceinline__ double sip_p(bool capped, const SipRow& ri, float s) {
    if (capped || ri.mode == 0) return 1.0;
    if (ri.mode == 1) return ri.c;
    return ri.c * fixed_point(s);
}

// Smallest integer T >= 1 with fl(c * T) >= 1 for the IEEE double product,
// capped at 2^53. fl(c * q) is non-decreasing in q, so for an integer q,
// fl(c * q) >= 1 exactly when q >= T. ceil(fl(1 / c)) lies within two of T,
// so a few exact integer steps in double find it.
__device__ __forceinline__ double cap_threshold(double c) {
    double t = ceil(1.0 / c);
    if (!(t < 0x1.0p53)) t = 0x1.0p53;
    if (t < 1.0) t = 1.0;
    // at most a few steps each (c is uniform, so are the exits)
    for (int i = 0; i < 4 && t > 1.0 && c * (t - 1.0) >= 1.0; ++i) t -= 1.0;
    for (int i = 0; i < 4 && t < 0x1.0p53 && c * t < 1.0; ++i) t += 1.0;
    return t;
}

// Smallest fp32 value s with s >= x (x > 0 and finite). For an fp32 score s
// and an integer T, floor(s * 2^52) >= T exactly when s >= this of T * 2^-52.
__device__ __forceinline__ float fp32_at_least(double x) {
    float f = static_cast<float>(x);
    if (static_cast<double>(f) < x) f = __uint_as_float(__float_as_uint(f) + 1u);
    return f;
}

// ---------------------------------------------------------------------------
// SIP probabilities and draws [hamidun, SIP paragraph; edumints, SIP item]:
// capped water-filling in exact fixed point (q_j = floor(s_j 2^52), exact
// sums, IEEE double division and product), then one Poisson draw per block.
// One workgroup of NT threads per plan row. Lane l of wave w owns the block
// pairs (2i, 2i+1) with i = i0(w, k) + l for passes k = 0, 1, ...: with
// MAXP > 0 the wave covers one contiguous range of 64 MAXP pairs
// (i0 = 64 (MAXP w + k)) and keeps their scores in registers (rows of up to
// 2 NT MAXP blocks); otherwise i0 = NT k + 64 w and every pass re-reads the
// scores from global memory. With contiguous ranges the blocks a round caps
// (neighbours in the video grid, hence in block order) fall in few waves,
// and a wave with none of them skips the round's pass.
//
// A round of the water-filling caps the still-active blocks with
// fl(c q_j) >= 1, i.e. q_j >= T(c) (cap_threshold), i.e. s_j >= thr(c) for
// the fp32 threshold fp32_at_least(T 2^-52). The capped set after any round
// is therefore {s_j >= thr_min}, thr_min the smallest threshold of a round
// that capped something, and a round's new caps are the blocks with
// thr <= s_j < thr_min: one fp32 comparison per block and round, and no
// per-block cap state. The row's outcome (mode, c, thr_min) goes to rowinfo,
// its keep mask (one bit per block, from the Philox draws) to keepmask and
// its cap mask (s_j >= thr_min) to capmask, so the fill kernel reads the
// score only of kept blocks that are not capped.
// ---------------------------------------------------------------------------
// NT threads per row (the launcher uses 512 or 768): with fewer threads the
// per-round work that every wave repeats (the threshold, the block
// reduction, its barriers) is shared by fewer waves, at the cost of more
// scores held per thread. Up to 20 pairs per thread the kernel is built for
// three workgroups per CU (6 waves per SIMD, at most 80 VGPRs): at 20 pairs
// this spills 40 bytes per lane, but the third workgroup hides more of the
// latency of the rounds' reductions than the spill costs (2.42 against
// 2.65 ms on 40 x 591 rows of 18,900 blocks); at 32 pairs the scores alone
// fill most of the 80 registers, and that tier keeps two workgroups.
//
// sip_row is the work of one row, for a workgroup of NT threads: load_pair(i)
// gives the scores of blocks 2i and 2i+1 (-1 past M: never capped, never
// kept), and on_kept(j, s_j) is called for every kept block j whose p
// depends on its score (not capped, mode 2): the blocks whose score the fill
// kernel reads. redd and redi hold 32 reduction slots ([16, 32): rounds 0,
// 2, ...; [0, 16): block_sum, rounds 1, 3, ...), redu NT/64.
template <int NT, int MAXP, typename LoadPair, typename OnKept>
__device__ __forceinline__ void sip_row(int64_t row, LoadPair&& load_pair, OnKept&& on_kept,
                                        int64_t H, int64_t QB, int64_t M, int64_t budget,
                                        uint64_t seed, int sampling,
                                        uint64_t* __restrict__ capmask,
                                        uint64_t* __restrict__ keepmask,
                                        SipRow* __restrict__ rowinfo,
                                        int64_t* __restrict__ counts,
                                        PlanStatus* __restrict__ status, double* redd, int* redi,
                                        uint64_t* redu) {
    constexpr int kSipPairsPerPass = NT;                 // block pairs per pass
    static_assert(NT / 64 <= 16, "reduction slots");
    const int64_t words = (M + 63) / 64;
    uint64_t* km = keepmask + row * words;
    uint64_t* cm = capmask + row * words;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: pass offsets in scalar registers
    const int M32 = static_cast<int>(M);                  // M < 2^19
    const int npairs = (M32 + 1) / 2;
    const int npass = (npairs + kSipPairsPerPass - 1) / kSipPairsPerPass;
    // register copies of the thread's pairs (two plain arrays so that they
    // stay in registers)
    // (at most 32 floats each: longer arrays the compiler leaves in scratch
    // memory)
    static_assert(MAXP <= 32, "register-resident pairs per thread");
    float sx[MAXP > 0 ? MAXP : 1], sy[MAXP > 0 ? MAXP : 1];
    auto get_pair = [&](int k) { return make_float2(sx[k], sy[k]); };
    auto set_pair = [&](int k, float2 v) { sx[k] = v.x; sy[k] = v.y; };
    // First pair of the wave's pass k (a multiple of 64): pbase + step k.
    // Written as one base plus constants so that nothing per pass stays
    // live (the lane's pair is one register plus an immediate; a pass lies
    // within the row iff step k < prem).
    constexpr int kPassStep = MAXP > 0 ? 64 : kSipPairsPerPass;
    const int pbase = MAXP > 0 ? 64 * MAXP * wave : 64 * wave;
    const int prem = npairs - pbase;
    const int ibase = pbase + lane;
    auto in_row = [&](int k) { return kPassStep * k < prem; };
    auto pair_at = [&](int k) {
        if constexpr (MAXP > 0) return get_pair(k);
        else return load_pair(ibase + kPassStep * k);
    };

    FixedSum sum;
    int bad = 0;
    float vmax = -1.0f;            // largest score of this thread not yet capped
    auto add_score = [&](float v, int j) {
        if (j >= M32) return;
        if (!(v >= 0.0f && v <= 1.0f)) bad = 1;
        else sum.add(v);
        vmax = fmaxf(vmax, v);
    };
    if constexpr (MAXP > 0) {
        // every load first (the scores stay in these registers anyway), so
        // their latencies overlap; then the sums
#pragma unroll
        for (int k = 0; k < MAXP; ++k) {
            const int i = ibase + kPassStep * k;
            set_pair(k, in_row(k) ? load_pair(i) : make_float2(-1.0f, -1.0f));
        }
#pragma unroll
        for (int k = 0; k < MAXP; ++k) {
            const int i = ibase + kPassStep * k;
            const float2 v = get_pair(k);
            add_score(v.x, 2 * i);
            add_score(v.y, 2 * i + 1);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        for (int k = 0; k < npass; ++k) {
            const int i = ibase + kPassStep * k;
            const float2 v = load_pair(i);
            add_score(v.x, 2 * i);
            add_score(v.y, 2 * i + 1);
        }
    }
    const double total = block_sum(sum.value(), redd);
    const int nbad = block_sum(bad, redi);
    if (nbad != 0 || total >= 0x1.0p53) {
        if (tid == 0) {
            status->bad_scores = 1;
            counts[row] = 0;
            rowinfo[row].mode = 0;
            rowinfo[row].c = 0.0;
            rowinfo[row].thr = INFINITY;
        }
        return;
    }

    int64_t taken = 0, n_active = M;
    double S = total;
    float thr_min = INFINITY;
    SipRow ri;
    int round = 0;
    for (;;) {
        const int64_t left = budget - taken;
        if (left >= n_active) { ri.mode = 0; ri.c = 1.0; break; }
        if (S == 0.0) {
            ri.mode = 1;
            ri.c = static_cast<double>(left) / static_cast<double>(n_active);
            break;
        }
        const double c = static_cast<double>(left) / S;
        const float thr = fp32_at_least(cap_threshold(c) * 0x1.0p-52);
        int ncap = 0;
        FixedSum scap;
        // If this round caps anything, thr < thr_min and thr becomes the new
        // thr_min, so the largest score below thr (m) is the next vmax; if
        // it caps nothing the rounds end and vmax is not read again.
        float m = -1.0f;
        auto test = [&](float v) {
            // opaque copy: keeps the conversions of every block from being
            // hoisted out of the rounds loop (64 live doubles otherwise)
            asm volatile("" : "+v"(v));
            if (v >= thr) {
                if (v < thr_min) {
                    ++ncap;
                    scap.add(v);
                }
            } else {
                m = fmaxf(m, v);
            }
        };
        // a wave none of whose uncapped scores reaches thr has no new cap,
        // and its vmax stays the largest score below the next thr_min
        if constexpr (MAXP > 0) {
            if (__builtin_amdgcn_ballot_w64(vmax >= thr) != 0) {
#pragma unroll
                for (int k = 0; k < MAXP; ++k) {
                    const float2 v = get_pair(k);
                    test(v.x);
                    test(v.y);
                    __builtin_amdgcn_sched_barrier(0);
                }
                vmax = m;
            }
        } else {
            for (int k = 0; k < npass; ++k) {
                const float2 v = pair_at(k);
                test(v.x);
                test(v.y);
            }
        }
        // both round totals in one block reduction (the fixed-point sums are
        // integers below 2^53, exact in any order)
        int tcap;
        double tsum;
        // the first round takes the second slot set: block_sum's slots may
        // still be read by waves that have not yet left it
        const int slot = (round & 1) ? 0 : 16;
        ++round;
        block_sum2(ncap, scap.value(), redi + slot, redd + slot, tcap, tsum);
        if (tcap == 0) { ri.mode = 2; ri.c = c; break; }
        taken += tcap;
        n_active -= tcap;
        S -= tsum;
        thr_min = fminf(thr_min, thr);
    }
    ri.thr = thr_min;

    const int64_t bidx = row / QB;
    const int64_t r = row - bidx * QB;
    const int64_t h = bidx % H;
    const int64_t b = bidx / H;
    int kept = 0;
    // In pass k wave w's lanes hold the pairs of blocks [2 i_0, 2 i_0 + 128)
    // (i_0 = pbase + step k, the pair of lane 0), i.e. mask words
    // w0 = i_0 / 32 and w0 + 1. Opaque copies of the bases: the pass offsets
    // are recomputed here, not kept live from the loads (registers).
    int ibase_d = ibase, prem_d = prem;
    asm volatile("" : "+v"(ibase_d), "+s"(prem_d));
    auto in_row_d = [&](int k) { return kPassStep * k < prem_d; };
    // The pass's keep and cap bits leave as mask words in block order.
    auto emit = [&](int k, bool keep0, bool keep1, bool cap0, bool cap1) {
        // Bit b of word w0 is block 2 (i_0 + b/2) + (b & 1), held by lane b/2
        // (of word w0 + 1: lane 32 + b/2). Lane b fetches that lane's four
        // bits and the ballots give the words in block order.
        const int packed = (keep0 ? 1 : 0) | (keep1 ? 2 : 0) | (cap0 ? 4 : 0) | (cap1 ? 8 : 0);
        const int f_lo = __builtin_amdgcn_ds_bpermute((lane >> 1) << 2, packed);
        const int f_hi = __builtin_amdgcn_ds_bpermute((32 + (lane >> 1)) << 2, packed);
        const int sh = lane & 1;
        const uint64_t k_lo = __ballot((f_lo >> sh) & 1), k_hi = __ballot((f_hi >> sh) & 1);
        const uint64_t c_lo = __ballot((f_lo >> (2 + sh)) & 1), c_hi = __ballot((f_hi >> (2 + sh)) & 1);
        if (lane == 0) {
            const int w0 = pbase / 32 + (kPassStep / 32) * k;
            if (w0 < words) {
                km[w0] = k_lo;
                cm[w0] = c_lo;
            }
            if (w0 + 1 < words) {
                km[w0 + 1] = k_hi;
                cm[w0 + 1] = c_hi;
            }
        }
        kept += (keep0 ? 1 : 0) + (keep1 ? 1 : 0);
    };
    if (sampling == kSamplingPoisson) {
        // one Bernoulli(p) per block
        auto draw = [&](int k, float2 v) {
            const int i = ibase_d + kPassStep * k;
            double u0 = 1.0, u1 = 1.0;
            sip_uniform_pair(seed, b, h, r, i, u0, u1);
            const bool cap0 = v.x >= thr_min, cap1 = v.y >= thr_min;
            const bool keep0 = 2 * i < M32 && u0 < sip_p(cap0, ri, v.x);
            const bool keep1 = 2 * i + 1 < M32 && u1 < sip_p(cap1, ri, v.y);
            if (ri.mode == 2) {
                if (keep0 && !cap0) on_kept(2 * i, v.x);
                if (keep1 && !cap1) on_kept(2 * i + 1, v.y);
            }
            emit(k, keep0, keep1, cap0, cap1);
        };
        if constexpr (MAXP > 0) {
#pragma unroll
            for (int k = 0; k < MAXP; ++k) {
                if (in_row_d(k)) draw(k, get_pair(k));
                // one pair's Philox at a time: keeps the register count low
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            for (int k = 0; k < npass; ++k) draw(k, pair_at(k));
        }
    } else {
        // Fixed-size design: sizes P_j = floor(p_j 2^40), exact integer
        // prefix sums in block order, one uniform U per row; block j is
        // taken iff a point U + k 2^40 falls in [C_{j-1}, C_j).
        const uint64_t U = sys_uniform(seed, b, h, r);
        struct PairSizes { uint64_t p0, p1; bool cap0, cap1; };
        auto sizes = [&](int k, float2 v) {
            const int i = ibase_d + kPassStep * k;
            PairSizes z;
            z.cap0 = v.x >= thr_min;
            z.cap1 = v.y >= thr_min;
            z.p0 = (2 * i < M32) ? sys_size(sip_p(z.cap0, ri, v.x)) : 0;
            z.p1 = (2 * i + 1 < M32) ? sys_size(sip_p(z.cap1, ri, v.y)) : 0;
            return z;
        };
        // pass k given the prefix before the pair of lane 0 (wave-uniform)
        auto take = [&](int k, float2 v, const PairSizes& z, uint64_t before, uint64_t incl) {
            const uint64_t c_prev = before + incl - (z.p0 + z.p1);
            const uint64_t c0 = c_prev + z.p0, c1 = c0 + z.p1;
            const uint64_t n_prev = sys_points_below(c_prev, U), n0 = sys_points_below(c0, U);
            const bool keep0 = n0 > n_prev, keep1 = sys_points_below(c1, U) > n0;
            if (ri.mode == 2) {
                const int i = ibase_d + kPassStep * k;
                if (keep0 && !z.cap0) on_kept(2 * i, v.x);
                if (keep1 && !z.cap1) on_kept(2 * i + 1, v.y);
            }
            emit(k, keep0, keep1, z.cap0, z.cap1);
        };
        if constexpr (MAXP > 0) {
            // the wave's range is contiguous: its prefix is the earlier
            // waves' totals, then pass by pass within the wave
            uint64_t wt = 0;
#pragma unroll
            for (int k = 0; k < MAXP; ++k) {
                if (in_row_d(k)) {
                    const PairSizes z = sizes(k, get_pair(k));
                    wt += z.p0 + z.p1;
                }
            }
            wt = wave_sum_u64(wt);
            if (lane == 0) redu[wave] = wt;
            __syncthreads();
            uint64_t before = 0;
            for (int w2 = 0; w2 < wave; ++w2) before += redu[w2];
#pragma unroll
            for (int k = 0; k < MAXP; ++k) {
                if (in_row_d(k)) {
                    const float2 v = get_pair(k);
                    const PairSizes z = sizes(k, v);
                    const uint64_t incl = wave_scan_u64(z.p0 + z.p1);
                    take(k, v, z, before, incl);
                    before += wave_last_u64(incl);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            // pass k covers pairs NT k .. NT k + NT - 1 across the waves
            uint64_t run = 0;
            for (int k = 0; k < npass; ++k) {
                const float2 v = pair_at(k);
                const PairSizes z = sizes(k, v);
                const uint64_t incl = wave_scan_u64(z.p0 + z.p1);
                if (lane == 63) redu[wave] = incl;
                __syncthreads();
                uint64_t before = run, tot = 0;
                for (int w2 = 0; w2 < NT / 64; ++w2) {
                    const uint64_t t = redu[w2];
                    if (w2 < wave) before += t;
                    tot += t;
                }
                take(k, v, z, before, incl);
                run += tot;
                __syncthreads();
            }
        }
    }
    const int tk = block_sum(kept, redi);
    if (tid == 0) {
        counts[row] = tk;
        rowinfo[row] = ri;
    }
}

// The SIP count of plan row blockIdx.x from its scores in global memory.
template <int NT, int MAXP>
__global__ __launch_bounds__(NT, (MAXP > 0 && MAXP <= 20) ? 6 : 4) void sip_count_kernel(
    const float* __restrict__ scores, int64_t H, int64_t QB, int64_t M, int64_t budget,
    uint64_t seed, int sampling, uint64_t* __restrict__ capmask, uint64_t* __restrict__ keepmask,
    SipRow* __restrict__ rowinfo, int64_t* __restrict__ counts, PlanStatus* __restrict__ status) {
    __shared__ double redd[32];
    __shared__ int redi[32];
    __shared__ uint64_t redu[NT / 64];
    const int64_t row = blockIdx.x;
    const float* sg = scores + row * M;
    const int M32 = static_cast<int>(M);                  // M < 2^19
    auto load_pair = [&](int i) {
        const int j = 2 * i;
        return make_float2(j < M32 ? sg[j] : -1.0f, j + 1 < M32 ? sg[j + 1] : -1.0f);
    };
    sip_row<NT, MAXP>(row, load_pair, [](int, float) {}, H, QB, M, budget, seed, sampling,
                      capmask, keepmask, rowinfo, counts, status, redd, redi, redu);
}

// ---------------------------------------------------------------------------
// Score pass 2 and the SIP count fused [hamidun, IBCS and SIP paragraphs]:
// the scores of a query block go from the matrix products straight to its
// water-filling and draws, without a round trip through memory. One
// workgroup of kFusedThreads threads per pair of query blocks (r, r+1) of a
// head, for plans of at most 8 clusters and rows of at most kFusedMaxBlocks
// KV blocks: the pair's two score rows sit in LDS (at most 158 KB).
//
// The scores are the two-pass kernel's bit for bit: the same block floating
// point digits (the centroid exponent is taken over the same group of
// 32 / CP query blocks, CP the two-pass kernel's cluster slots per query
// block), the same exact int32 digit products, the same fp32 combination,
// bias (from pass 1's chunk statistics) and order of the sum over clusters.
// The contraction runs on the 16x16x64 int8 MFMA: A = the pair's 16
// centroid slots (query block r + s/8, cluster s%8), B = 16 keys; D layout:
// lane l holds key l%16 and slots 4 (l/16) + i, i < 4, i.e. the four
// clusters of one half of the query block's clusters, whose partial sum the
// lane sixteen apart completes. Each wave takes every 16th 16-key tile, so
// the workgroup reads its head's key digits front to back once; the tile's
// digits (the tile-major copy the mean-key kernel writes, one contiguous
// 1 KB run per operand load) go straight to registers (no LDS: the rows
// fill it), two tiles alternating so that one loads while the other is
// computed.
//
// Then each row's SIP count (sip_row) runs on all the workgroup's waves
// with the scores read from LDS; the only scores written to memory are
// those of kept blocks whose p depends on them, at their positions in the
// row (the fill kernel reads no others).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kFusedThreads, 1) void scores_sip_kernel(
    const float* __restrict__ cent, const float* __restrict__ w, const int8_t* __restrict__ kqt,
    const int* __restrict__ kx, const float* __restrict__ sbias, int64_t H, int64_t QB, int64_t M,
    int C, float scale_log2, int64_t budget, uint64_t seed, int sampling,
    float* __restrict__ scores, uint64_t* __restrict__ capmask, uint64_t* __restrict__ keepmask,
    SipRow* __restrict__ rowinfo, int64_t* __restrict__ counts, PlanStatus* __restrict__ status) {
    constexpr int NT = kFusedThreads;
    // register-resident pairs per thread in the SIP phase: rows up to
    // 2 NT kFusedSipPairs blocks (kFusedMaxBlocks fits)
    constexpr int kFusedSipPairs = 10;
    static_assert(2 * NT * kFusedSipPairs >= kFusedMaxBlocks, "fused rows fit the SIP registers");
    constexpr int NSTEP = D / 64;                   // MFMA k-steps (64 channels each)
    constexpr int NW = NT / 64;
    typedef int intx4 __attribute__((ext_vector_type(4)));
    __shared__ float srow[2][kFusedMaxBlocks];
    __shared__ double redd[32];
    __shared__ int redi[32];
    __shared__ uint64_t redu[NW];
    __shared__ float wmax[NW];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t bh = blockIdx.y;
    const int64_t r = 2 * static_cast<int64_t>(blockIdx.x);
    const int M32 = static_cast<int>(M);

    // Exponent of the centroids: the largest |c| over the query blocks of
    // the two-pass kernel's wave group (32 / CP of them, aligned; an even r
    // and its successor lie in the same group) and their C clusters.
    const int cp = C <= 1 ? 1 : C <= 2 ? 2 : C <= 4 ? 4 : 8;
    const int64_t grp = 32 / cp;
    const int64_t g0 = (r / grp) * grp;
    const int64_t gn = ((g0 + grp < QB) ? grp : QB - g0) * C * D;
    float amax = 0.0f;
    {
        // gn is a multiple of D, the rows 256-byte aligned: float4 reads
        const float4* gsrc = reinterpret_cast<const float4*>(cent + (bh * QB + g0) * C * D);
        for (int64_t e = tid; e < gn / 4; e += NT) {
            const float4 x = gsrc[e];
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
        if (lane == 0) wmax[wave] = amax;
        __syncthreads();
        amax = wmax[0];
        for (int k = 1; k < NW; ++k) amax = fmaxf(amax, wmax[k]);
    }
    const int ex = bfp_exponent(amax);
    const float rowf = ldexpf(scale_log2, ex - 28);

    // A operands: slot s = lane % 16, channels 64 st + 16 (lane / 16) .. +16.
    intx4 a2[NSTEP], a1[NSTEP], a0[NSTEP];
    {
        const int slot = lane & 15;
        const int64_t rs = r + (slot >> 3);
        const int m = slot & 7;
        const bool ok = rs < QB && m < C;
        // an empty slot reads centroid 0 of block r (in bounds) and uses zeros:
        // unconditional vector loads, all in flight together
        const float4* src = reinterpret_cast<const float4*>(
            cent + ((bh * QB + (ok ? rs : r)) * C + (ok ? m : 0)) * D + (lane >> 4) * 16);
        float4 xv[NSTEP][4];
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
#pragma unroll
            for (int u = 0; u < 4; ++u) xv[st][u] = src[st * 16 + u];
        }
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
            int8_t h2[16], h1[16], h0[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float4 x4 = xv[st][e >> 2];
                const float x = (e & 3) == 0 ? x4.x : (e & 3) == 1 ? x4.y : (e & 3) == 2 ? x4.z : x4.w;
                bfp_digits(ok ? x : 0.0f, ex, h2[e], h1[e], h0[e]);
            }
            __builtin_memcpy(&a2[st], h2, 16);
            __builtin_memcpy(&a1[st], h1, 16);
            __builtin_memcpy(&a0[st], h0, 16);
        }
    }
    // this lane's output slots 4 (lane / 16) + i: query block r + lane / 32,
    // clusters 4 ((lane / 16) % 2) + i
    float bias[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t rb = r + (lane >> 5);
        const int mb = 4 * ((lane >> 4) & 1) + i;
        bias[i] = (rb < QB && mb < C) ? sbias[(bh * QB + rb) * C + mb] : -INFINITY;
    }

    const int ntile = (M32 + 15) / 16;
    const int8_t* kt = kqt + bh * ntile * (3 * D * 16) + lane * 16;
    const int* kxb = kx + bh * M;
    const int kc = lane & 15;
    const bool writer = ((lane >> 4) & 1) == 0;
    float* sr = srow[lane >> 5];
    // digits of this lane's key of tile t (tile-major digits: each operand a
    // contiguous 1 KB run; tiles past the row re-read the last tile, keys
    // past M are never stored)
    struct Tile { intx4 b2[NSTEP], b1[NSTEP], b0[NSTEP]; int kexp; };
    auto fetch = [&](int t, Tile& tl) __attribute__((always_inline)) {
        const int tc = min(t, ntile - 1);
        const int8_t* kp = kt + static_cast<int64_t>(tc) * (3 * D * 16);
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
            tl.b2[st] = *reinterpret_cast<const intx4*>(kp + st * 1024);
            tl.b1[st] = *reinterpret_cast<const intx4*>(kp + (NSTEP + st) * 1024);
            tl.b0[st] = *reinterpret_cast<const intx4*>(kp + (2 * NSTEP + st) * 1024);
        }
        tl.kexp = kxb[min(tc * 16 + kc, M32 - 1)];
    };
    auto compute = [&](int t, const Tile& tl) __attribute__((always_inline)) {
        intx4 o22 = intx4{}, o21 = intx4{}, o20 = intx4{};
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
            o22 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2[st], tl.b2[st], o22, 0, 0, 0);
            o21 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2[st], tl.b1[st], o21, 0, 0, 0);
            o20 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2[st], tl.b0[st], o20, 0, 0, 0);
            o21 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1[st], tl.b2[st], o21, 0, 0, 0);
            o20 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1[st], tl.b1[st], o20, 0, 0, 0);
            o20 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0[st], tl.b2[st], o20, 0, 0, 0);
        }
        // the two-pass kernel's combination and key factor, then its sum over
        // the half's clusters in cluster order, then the two halves
        const float cf = ldexpf(rowf, tl.kexp);
        float pr = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int lo = (o21[i] << 8) + o20[i];
            const float x = fmaf(static_cast<float>(o22[i]), 65536.0f, static_cast<float>(lo));
            pr += __builtin_amdgcn_exp2f(fmaf(x, cf, bias[i]));
        }
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_int(pr), __float_as_int(pr),
                                                          false, false);
        const float sc = __int_as_float(sw[0]) + __int_as_float(sw[1]);
        const int j = t * 16 + kc;
        if (writer && j < M32) sr[j] = sc;
    };
    // two tiles in registers, alternately loaded and consumed: a tile's loads
    // are in flight while the other tile is computed. The loads are
    // unconditional (past the row they re-read its last key, unused), so
    // that every path leaves them in the same order and each compute waits
    // only for its own tile.
    Tile ta, tb;
    fetch(wave, ta);
    for (int t = wave; t < ntile; t += 2 * NW) {
        fetch(t + NW, tb);
        compute(t, ta);
        fetch(t + 2 * NW, ta);
        if (t + NW < ntile) compute(t + NW, tb);
    }
    __syncthreads();

    for (int q = 0; q < 2; ++q) {
        const int64_t rq = r + q;
        if (rq >= QB) break;
        const int64_t row = bh * QB + rq;
        const float* ls = srow[q];
        float* so = scores + row * M;
        auto load_pair = [&](int i) {
            const int j = 2 * i;
            return make_float2(j < M32 ? ls[j] : -1.0f, j + 1 < M32 ? ls[j + 1] : -1.0f);
        };
        sip_row<NT, kFusedSipPairs>(row, load_pair, [&](int j, float v) { so[j] = v; }, H, QB,
                                    M, budget, seed, sampling, capmask, keepmask, rowinfo,
                                    counts, status, redd, redi, redu);
    }
}

// Exclusive scan of the per-row counts into rowptr[0..rows]; one workgroup.
__global__ __launch_bounds__(1024) void scan_kernel(const int64_t* __restrict__ counts,
                                                    int64_t rows, int64_t* __restrict__ rowptr,
                                                    PlanStatus* __restrict__ status) {
    __shared__ int64_t wsum[16];
    __shared__ int64_t carry_s;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) carry_s = 0;
    __syncthreads();
    for (int64_t base = 0; base < rows; base += 1024) {
        const int64_t i = base + tid;
        const int64_t v = (i < rows) ? counts[i] : 0;
        int64_t incl = v;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int64_t t = __shfl_up(incl, off);
            if (lane >= off) incl += t;
        }
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        int64_t woff = 0;
        for (int k = 0; k < wave; ++k) woff += wsum[k];
        const int64_t carry = carry_s;
        if (i < rows) rowptr[i] = carry + woff + incl - v;
        __syncthreads();
        if (tid == 1023) carry_s = carry + woff + incl;
        __syncthreads();
    }
    if (tid == 0) {
        rowptr[rows] = carry_s;
        status->nnz = carry_s;
    }
}

// Fill the CSR row from the keep mask: ascending kept block indices, fp32
// log-weights -ln p (+0 for p = 1), and p. The row's mask words are taken in
// chunks of 256: thread t first counts word t of the chunk and a block-wide
// exclusive scan gives every word's first output position (in LDS); then
// each wave expands 64 of the chunk's words one at a time, lane l handling
// bit l, so a word's kept blocks are written by consecutive lanes to
// consecutive positions (v_mbcnt gives each lane its rank in the word).
// Blocks with p = 1 (capped, or every block in mode 0) and mode 1's uniform
// p are written at once. The kept blocks of mode 2 that are not capped
// (about one per word) need their score, p = c * q and an fp64 logarithm:
// they are queued per wave in LDS and handled 64 at a time, one per lane,
// so each logarithm instruction serves a full wave instead of one lane.
__global__ __launch_bounds__(256) void sip_fill_kernel(
    const float* __restrict__ scores, int64_t M, const uint64_t* __restrict__ capmask,
    const uint64_t* __restrict__ keepmask, const SipRow* __restrict__ rowinfo,
    const int64_t* __restrict__ rowptr, int sampling, int32_t* __restrict__ idx,
    float* __restrict__ logw, double* __restrict__ p_out) {
    __shared__ int wtot[4];
    __shared__ int word_pos[256];
    __shared__ int64_t q_at[4][64];                    // queued output positions, per wave
    __shared__ int q_j[4][64];                         // and their block indices
    const int64_t row = blockIdx.x;
    const float* sg = scores + row * M;
    const int words = static_cast<int>((M + 63) / 64);
    const uint64_t* cm = capmask + row * static_cast<int64_t>(words);
    const uint64_t* km = keepmask + row * static_cast<int64_t>(words);
    const SipRow ri = rowinfo[row];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // The plan's p: the design's inclusion probability (under the fixed-size
    // design, p rounded down to a multiple of 2^-40).
    auto incl_p = [&](double p) {
        return (sampling == kSamplingSystematic) ? floor(p * 0x1.0p40) * 0x1.0p-40 : p;
    };
    // p and -ln p of a block that is neither capped nor queued
    const double p_direct = incl_p((ri.mode == 1) ? ri.c : 1.0);
    const float lw_direct = (p_direct == 1.0) ? 0.0f : static_cast<float>(-log(p_direct));
    int nq = 0;                                        // queue length (wave-uniform)
    auto flush = [&]() {
        if (lane < nq) {
            const int64_t at = q_at[wave][lane];
            const int j = q_j[wave][lane];
            const double p = incl_p(sip_p(false, ri, sg[j]));
            logw[at] = (p == 1.0) ? 0.0f : static_cast<float>(-log(p));
            p_out[at] = p;
        }
        nq = 0;
    };
    int64_t pos = rowptr[row];
    for (int base = 0; base < words; base += 256) {
        const int w = base + tid;
        // thread t holds word t of the chunk; the expansion below takes the
        // words of its wave from their lanes (no dependent reloads)
        const uint64_t kw_own = (w < words) ? km[w] : 0ull;
        const uint64_t cw_own = (w < words) ? cm[w] : 0ull;
        const int pc = __popcll(kw_own);
        int incl = pc;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(incl, off);
            if (lane >= off) incl += t;
        }
        if (lane == 63) wtot[wave] = incl;
        __syncthreads();
        int woff = 0, tot = 0;
        for (int k = 0; k < 4; ++k) {
            if (k < wave) woff += wtot[k];
            tot += wtot[k];
        }
        word_pos[tid] = woff + incl - pc;
        __syncthreads();
        const int wend = min(64, words - base - 64 * wave);
        for (int u = 0; u < wend; ++u) {
            const int wl = 64 * wave + u;                 // word within the chunk
            const uint64_t kw = readlane_u64(kw_own, u);  // word wl, wave-uniform
            if (kw == 0) continue;
            const uint64_t cw = readlane_u64(cw_own, u);
            const uint64_t qw = (ri.mode == 2) ? (kw & ~cw) : 0ull;   // blocks to queue
            const int nqw = __popcll(qw);
            if (nq + nqw > 64) flush();
            if ((kw >> lane) & 1ull) {
                const int rank = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(kw >> 32),
                                 __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(kw), 0));
                const int64_t at = pos + word_pos[wl] + rank;
                const int j = (base + wl) * 64 + lane;
                idx[at] = j;
                if ((qw >> lane) & 1ull) {
                    const int qr = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(qw >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(qw), 0));
                    q_at[wave][nq + qr] = at;
                    q_j[wave][nq + qr] = j;
                } else {
                    const bool capped = (cw >> lane) & 1ull;
                    logw[at] = capped ? 0.0f : lw_direct;
                    p_out[at] = capped ? 1.0 : p_direct;
                }
            }
            nq += nqw;
        }
        flush();
        pos += tot;
        __syncthreads();
    }
}

template <typename F>
hipError_t launch_checked(F&& f) {
    f();
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mean_keys(const void* k, Dtype dt, int64_t BH, int64_t N, int d,
                            float* kbar, int8_t* kq, int8_t* kqt, int* kx, hipStream_t s) {
    const int64_t M = N / kKvBlock;
    const int64_t chunks = BH * M * (d / 4);
    const int threads = 256;                    // a multiple of d/4: blocks never straddle
    const int64_t blocks = (chunks + threads - 1) / threads;
    if (blocks == 0) return hipSuccess;
    return launch_checked([&] {
        if (dt == kBF16)
            hipLaunchKernelGGL(mean_keys_kernel<uint16_t>, dim3(blocks), dim3(threads), 0, s,
                               static_cast<const uint16_t*>(k), kbar, kq, kqt, kx, chunks, M, d);
        else
            hipLaunchKernelGGL(mean_keys_kernel<float>, dim3(blocks), dim3(threads), 0, s,
                               static_cast<const float*>(k), kbar, kq, kqt, kx, chunks, M, d);
    });
}

template <typename T, int D>
static void launch_kmeans_t(const void* q, int64_t BH, int64_t N, int C, int iters, float* cent,
                            float* w, hipStream_t s) {
    const int64_t QB = (N + kQueryBlock - 1) / kQueryBlock;
    if (C <= 8)
        hipLaunchKernelGGL((kmeans_kernel<T, D, 4>), dim3(BH * QB), dim3(256), 0, s,
                           static_cast<const T*>(q), N, QB, C, iters, cent, w);
    else
        hipLaunchKernelGGL((kmeans_kernel<T, D, 8>), dim3(BH * QB), dim3(256), 0, s,
                           static_cast<const T*>(q), N, QB, C, iters, cent, w);
}

hipError_t launch_kmeans(const void* q, Dtype dt, int64_t BH, int64_t N, int d, int C,
                         int iters, float* cent, float* w, hipStream_t s) {
    return launch_checked([&] {
        if (dt == kBF16) {
            if (d == 128) launch_kmeans_t<uint16_t, 128>(q, BH, N, C, iters, cent, w, s);
            else launch_kmeans_t<uint16_t, 64>(q, BH, N, C, iters, cent, w, s);
        } else {
            if (d == 128) launch_kmeans_t<float, 128>(q, BH, N, C, iters, cent, w, s);
            else launch_kmeans_t<float, 64>(q, BH, N, C, iters, cent, w, s);
        }
    });
}

// Key chunking of the score passes: whole rows of keys when the
// (query-block group x head) grid alone fills the chip, else just enough
// even chunks for about kScoreMinGroups workgroups. Splitting costs a
// second read of every chunk's statistics, so it is kept for small grids.
constexpr int64_t kScoreMinGroups = 1024;

static void score_chunks(int64_t groups, int64_t M, int* chunk_tiles, int* nchunks) {
    const int64_t ntiles = (M + kScoreTile - 1) / kScoreTile;
    int64_t n = (kScoreMinGroups + groups - 1) / groups;
    if (n > ntiles) n = ntiles;
    if (n < 1) n = 1;
    *chunk_tiles = static_cast<int>((ntiles + n - 1) / n);
    *nchunks = static_cast<int>((ntiles + *chunk_tiles - 1) / *chunk_tiles);
}

static int64_t score_groups(int64_t BH, int64_t QB, int C) {
    const int cp = C <= 1 ? 1 : C <= 2 ? 2 : C <= 4 ? 4 : C <= 8 ? 8 : 16;
    const int64_t rows_per_wg = kScoreWaves * (32 / cp);
    return BH * ((QB + rows_per_wg - 1) / rows_per_wg);
}

int64_t score_partials(int64_t BH, int64_t QB, int64_t M, int C) {
    int ct = 0, nc = 0;
    score_chunks(score_groups(BH, QB, C), M, &ct, &nc);
    return BH * QB * C * nc;
}

template <int CP, int D>
static void launch_scores_cpd(const float* cent, const float* w, const int8_t* kq,
                              const int* kx, int64_t BH, int64_t QB, int64_t M, int C,
                              float2* part, float* sbias, float* scores, bool pass2,
                              hipStream_t s) {
    constexpr int rows_per_wg = kScoreWaves * (32 / CP);
    int chunk_tiles = 0, nchunks = 0;
    score_chunks(score_groups(BH, QB, C), M, &chunk_tiles, &nchunks);
    const dim3 grid(static_cast<unsigned>((QB + rows_per_wg - 1) / rows_per_wg),
                    static_cast<unsigned>(BH), static_cast<unsigned>(nchunks));
    const float scale_log2 = kLog2e / sqrtf(static_cast<float>(D));
    hipLaunchKernelGGL((scores_kernel<CP, D, false>), grid, dim3(256), 0, s, cent, w, kq, kx, QB,
                       M, C, chunk_tiles, nchunks, scale_log2, part, sbias, scores);
    const int64_t nb = BH * QB * C;
    hipLaunchKernelGGL(score_bias_kernel, dim3(static_cast<unsigned>((nb + 255) / 256)), dim3(256),
                       0, s, part, w, QB, C, nchunks, nb, sbias);
    if (pass2)
        hipLaunchKernelGGL((scores_kernel<CP, D, true>), grid, dim3(256), 0, s, cent, w, kq, kx,
                           QB, M, C, chunk_tiles, nchunks, scale_log2, part, sbias, scores);
}

template <int CP>
static void launch_scores_cp(const float* cent, const float* w, const int8_t* kq, const int* kx,
                             int64_t BH, int64_t QB, int64_t M, int d, int C, float2* part,
                             float* sbias, float* scores, bool pass2, hipStream_t s) {
    if (d == 128)
        launch_scores_cpd<CP, 128>(cent, w, kq, kx, BH, QB, M, C, part, sbias, scores, pass2, s);
    else
        launch_scores_cpd<CP, 64>(cent, w, kq, kx, BH, QB, M, C, part, sbias, scores, pass2, s);
}

hipError_t launch_scores(const float* cent, const float* w, const int8_t* kq, const int* kx,
                         int64_t BH, int64_t QB, int64_t M, int d, int C, float2* part,
                         float* sbias, float* scores, bool pass2, hipStream_t s) {
    return launch_checked([&] {
        auto go = [&](auto cp) {
            launch_scores_cp<decltype(cp)::value>(cent, w, kq, kx, BH, QB, M, d, C, part, sbias,
                                                  scores, pass2, s);
        };
        if (C <= 1) go(std::integral_constant<int, 1>{});
        else if (C <= 2) go(std::integral_constant<int, 2>{});
        else if (C <= 4) go(std::integral_constant<int, 4>{});
        else if (C <= 8) go(std::integral_constant<int, 8>{});
        else go(std::integral_constant<int, 16>{});
    });
}

hipError_t launch_scores_sip(const float* cent, const float* w, const int8_t* kqt, const int* kx,
                             const float* sbias, int64_t B, int64_t H, int64_t QB, int64_t M,
                             int d, int C, int64_t budget, uint64_t seed, int sampling,
                             float* scores, uint64_t* capmask, uint64_t* keepmask,
                             SipRow* rowinfo, int64_t* counts, PlanStatus* status,
                             hipStream_t s) {
    if (C < 1 || C > 8 || M > kFusedMaxBlocks || (d != 64 && d != 128)) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>((QB + 1) / 2), static_cast<unsigned>(B * H));
    return launch_checked([&] {
        if (d == 128)
            hipLaunchKernelGGL(scores_sip_kernel<128>, grid, dim3(kFusedThreads), 0, s, cent, w,
                               kqt, kx, sbias, H, QB, M, C, kLog2e / sqrtf(128.0f), budget, seed,
                               sampling, scores, capmask, keepmask, rowinfo, counts, status);
        else
            hipLaunchKernelGGL(scores_sip_kernel<64>, grid, dim3(kFusedThreads), 0, s, cent, w,
                               kqt, kx, sbias, H, QB, M, C, kLog2e / sqrtf(64.0f), budget, seed,
                               sampling, scores, capmask, keepmask, rowinfo, counts, status);
    });
}

hipError_t launch_sip_count(const float* scores, int64_t B, int64_t H, int64_t QB, int64_t M,
                            int64_t budget, uint64_t seed, int sampling, uint64_t* capmask,
                            uint64_t* keepmask,
                            SipRow* rowinfo, int64_t* counts, PlanStatus* status, hipStream_t s) {
    const int64_t rows = B * H * QB;
    // 512 threads per row, the scores of up to 20 pairs per thread in
    // registers (rows of up to 20,480 blocks); then 768 threads at 20 pairs
    // (up to 30,720 blocks: 6 waves per SIMD where 512 threads at 24 or 32
    // pairs run 4) and 512 at 32 (up to 32,768); longer rows re-read their
    // scores every pass. (Other shapes for the Wan2.1-like rows of 18,900
    // blocks were measured slower: 320 threads at 30 pairs 5.6 against
    // 3.8 ms before later changes; 768 at 13 and 1024 at 10 pairs 2.50 and
    // 2.73 against 2.35 ms.)
    const int64_t pairs = (M + 1) / 2;
    const int64_t npass = (pairs + 511) / 512;
    return launch_checked([&] {
#define ABSA_SIP_LAUNCH(NT, MP)                                                                  \
    hipLaunchKernelGGL((sip_count_kernel<NT, MP>), dim3(rows), dim3(NT), 0, s, scores, H, QB,   \
                       M, budget, seed, sampling, capmask, keepmask, rowinfo, counts, status)
        if (npass <= 8) ABSA_SIP_LAUNCH(512, 8);
        else if (npass <= 16) ABSA_SIP_LAUNCH(512, 16);
        else if (npass <= 20) ABSA_SIP_LAUNCH(512, 20);
        else if (pairs <= 768 * 20) ABSA_SIP_LAUNCH(768, 20);
        else if (npass <= 32) ABSA_SIP_LAUNCH(512, 32);
        else ABSA_SIP_LAUNCH(512, 0);
#undef ABSA_SIP_LAUNCH
    });
}

hipError_t launch_scan(const int64_t* counts, int64_t rows, int64_t* rowptr, PlanStatus* status,
                       hipStream_t s) {
    return launch_checked([&] {
        hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, counts, rows, rowptr, status);
    });
}

hipError_t launch_sip_fill(const float* scores, int64_t rows, int64_t M, const uint64_t* capmask,
                           const uint64_t* keepmask, const SipRow* rowinfo, const int64_t* rowptr,
                           int sampling, int32_t* idx, float* logw, double* p, hipStream_t s) {
    return launch_checked([&] {
        hipLaunchKernelGGL(sip_fill_kernel, dim3(rows), dim3(256), 0, s, scores, M, capmask,
                           keepmask, rowinfo, rowptr, sampling, idx, logw, p);
    });
}

}  // namespace absa
