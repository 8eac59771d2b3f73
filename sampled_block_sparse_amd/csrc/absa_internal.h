// Internal declarations shared by the host layer (absa.cpp) and the HIP
// kernel sources. Not part of the public interface (include/absa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace absa {

constexpr int kQueryBlock = 128;   // queries per plan row
constexpr int kKvBlock = 4;        // tokens per KV block
constexpr int kMaxClusters = 16;

enum Dtype : int { kBF16 = 0, kF32 = 1 };

// Sampling designs of the plan (values of absa_plan_params.sampling).
constexpr int kSamplingPoisson = 0;
constexpr int kSamplingSystematic = 1;

// Per-row outcome of the capped water-filling, written by the SIP count
// kernel and read by the fill kernel.
//   mode 0: every still-active block has p = 1
//   mode 1: every still-active block has p = left / n_active (all scores 0)
//   mode 2: every still-active block has p = c * q_j
// The capped blocks (p = 1) are exactly those with score >= thr (+inf when
// no block is capped).
struct SipRow {
    double c;          // mode 2 multiplier, or left/n_active for mode 1
    int32_t mode;
    float thr;
};

// Device-side status written at the end of the SIP count + scan and read
// back by the host in the plan's single synchronisation.
struct PlanStatus {
    int64_t nnz;
    int32_t bad_scores;   // a score outside [0,1] / NaN, or a row sum >= 2
    int32_t pad;
};

// kbar: fp32 means [BH, M, d], or null to skip them; kq: their block floating point int8 digits
// [BH, M, 3, d] (planes X2, X1, X0) and kx: the exponent of each mean [BH, M],
// the score kernel's operand; kqt, or null to skip it: the same digits
// tile-major for the fused score kernel ([BH, ceil(M/16), 3, d/64, 64 lanes,
// 16 bytes]: kqt_bytes).
hipError_t launch_mean_keys(const void* k, Dtype dt, int64_t BH, int64_t N, int d,
                            float* kbar, int8_t* kq, int8_t* kqt, int* kx, hipStream_t s);
inline int64_t kqt_bytes(int64_t BH, int64_t M, int d) { return BH * ((M + 15) / 16) * 16 * 3 * d; }

hipError_t launch_kmeans(const void* q, Dtype dt, int64_t BH, int64_t N, int d,
                         int C, int iters, float* cent, float* w, hipStream_t s);

// Number of float2 chunk statistics the score passes need (the part
// argument of launch_scores).
int64_t score_partials(int64_t BH, int64_t QB, int64_t M, int C);

// Pass 1 (chunk statistics into part), the bias of every (query block,
// centroid) from them (sbias, float [BH*QB*C]), then pass 2 (scores) unless
// pass2 = false (the fused kernel takes sbias instead).
hipError_t launch_scores(const float* cent, const float* w, const int8_t* kq, const int* kx,
                         int64_t BH, int64_t QB, int64_t M, int d, int C,
                         float2* part, float* sbias, float* scores, bool pass2, hipStream_t s);

// Score pass 2 fused with the SIP count: the same outputs as pass 2 and
// launch_sip_count, except that scores receives only the scores the fill
// kernel reads (kept blocks that are not capped). Needs C <= 8 and
// M <= kFusedMaxBlocks; sbias from launch_scores(..., pass2 = false), kqt
// from launch_mean_keys.
constexpr int kFusedThreads = 1024;
constexpr int64_t kFusedMaxBlocks = 20224;
hipError_t launch_scores_sip(const float* cent, const float* w, const int8_t* kqt, const int* kx,
                             const float* sbias, int64_t B, int64_t H, int64_t QB, int64_t M,
                             int d, int C, int64_t budget, uint64_t seed, int sampling,
                             float* scores, uint64_t* capmask, uint64_t* keepmask,
                             SipRow* rowinfo, int64_t* counts, PlanStatus* status,
                             hipStream_t s);

hipError_t launch_sip_count(const float* scores, int64_t B, int64_t H, int64_t QB,
                            int64_t M, int64_t budget, uint64_t seed, int sampling,
                            uint64_t* capmask,
                            uint64_t* keepmask, SipRow* rowinfo, int64_t* counts,
                            PlanStatus* status, hipStream_t s);

hipError_t launch_scan(const int64_t* counts, int64_t rows, int64_t* rowptr,
                       PlanStatus* status, hipStream_t s);

hipError_t launch_sip_fill(const float* scores, int64_t rows, int64_t M,
                           const uint64_t* capmask, const uint64_t* keepmask,
                           const SipRow* rowinfo,
                           const int64_t* rowptr, int sampling, int32_t* idx, float* logw,
                           double* p, hipStream_t s);

// Static scratch of the allocation-free attention call: three bf16 copies of
// fp32 inputs of at most kNoAllocMaxElems elements each. noalloc_scratch
// gives its address on the current device (looked up once per device).
constexpr int64_t kNoAllocMaxElems = int64_t(1) << 22;
hipError_t noalloc_scratch(uint16_t** out);

// fp32 -> bf16 (round to nearest even) of n elements, n a multiple of 8.
hipError_t launch_to_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s);

// Attention on bf16 q, k, v [B, H, N, d]; o is fp32 when out_f32, else bf16.
hipError_t launch_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o,
                            bool out_f32, int64_t B, int64_t H, int64_t N, int d,
                            const int64_t* rowptr, const int32_t* idx,
                            const float* logw, bool dense, hipStream_t s);

}  // namespace absa
