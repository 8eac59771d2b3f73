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
//     accumulators (converted to bf16), A = V^T read from a row-major V tile
//     in LDS with the gfx950 transpose read (ds_read_b64_tr_b16), addressed
//     so that its key order matches the accumulator layout of P: no lane
//     exchange and no transposed stores. O^T has the query in the lane's
//     column, so the online-softmax rescale is lane-local.
//   * Software pipeline with one barrier per tile: each wave issues tile
//     t+1's S^T MFMAs next to tile t's softmax, then tile t's P V MFMAs. Two
//     LDS buffers hold K and V of alternate tiles; K of tile t+2 is stored
//     just before the barrier and V after it, and the gather of tile t+3
//     into registers overlaps the whole next iteration. Two workgroups per CU. Block ids
//     and log-weights come through scalar loads; gather addresses are 32-bit
//     offsets from the head's base.
//   * Softmax per 4-key group: the group max of the raw products sets the
//     tile max with one FMA per group, each weight is exp2 of one FMA
//     (scale, log-weight and running max folded together), and the output
//     is rescaled only in tiles where some lane's running max grows.
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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

// Two floats to packed bf16 (round to nearest even): one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const floatx2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// Value of lane l^32 and of lane l combined: v_permlane32_swap exchanges the
// two 32-lane halves, so {r[0], r[1]} = {own, partner}.
__device__ __forceinline__ float half_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// The output is rescaled only in tiles where some lane's running max grows
// (a wave-uniform branch). Deferring the rescale until the max grows by more
// than a slack was measured: the largest weight of a row is then no longer
// exactly 1 in bf16, which raises the output error on concentrated attention
// for a gain below 1%, so the max is always exact.

// Per-lane prefetch registers for one tile: 16 bytes of K and of V at the
// same (key, channel) position of the lane's KV block.
template <int D, bool F32> struct TileRegs;
template <int D> struct TileRegs<D, false> {
    uint4 k[D / 32];
    uint4 v[D / 32];
    float lw[D / 32];
};
template <int D> struct TileRegs<D, true> {
    float4 k[D / 32][2];
    float4 v[D / 32][2];
    float lw[D / 32];
};

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

// gfx950 transpose read: within each group of 16 lanes, lane i receives
// element i%4 of the 8-byte rows addressed by lanes i/4, 4+i/4, 8+i/4 and
// 12+i/4 of its group.
__device__ __forceinline__ uint2 ds_read_tr16(const uint16_t* p) {
    const shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p));
    return __builtin_bit_cast(uint2, v);
}

// V tiles are stored row-major [key][channel] with 64-byte segments XOR-ed
// by a function of the key row, so that the transpose reads of 4 consecutive
// keys x 64 bytes hit distinct LDS banks.
template <int D> __device__ __forceinline__ int vseg_swizzle(int key) {
    return (D == 128) ? (key & 3) : ((key >> 1) & 1);
}

template <int D, bool F32, bool DENSE>
__global__ __launch_bounds__(256, 2) void attn_kernel(AttnParams P) {
    constexpr int KS = D + 8;                   // K tile row stride (bf16)
    constexpr int NP = D / 32;                  // loader passes per tile
    constexpr int LPB = D / 2;                  // lanes per KV block in a pass
    constexpr int BPP = 64 / LPB;               // blocks per pass per wave
    constexpr int NS = D / 16;                  // 16-channel MFMA steps
    constexpr int ND = D / 32;                  // 32-channel output blocks
    constexpr int ESZ = F32 ? 4 : 2;            // bytes per input element
    constexpr uint32_t BLOCK_BYTES = kKvBlock * D * ESZ;
    __shared__ __align__(16) uint16_t Ks[2][kTileKeys * KS];
    __shared__ __align__(16) uint16_t Vs[2][kTileKeys * D];
    __shared__ float lws[2][kTileBlocks];

    const int bid = blockIdx.x;
    const int64_t row = static_cast<int64_t>(bid % kXcds) * P.per_xcd + bid / kXcds;
    if (row >= P.rows) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int half = lane >> 5;

    const int64_t bh = row / P.QB;
    const int64_t r = row - bh * P.QB;
    const int64_t q0 = r * kQueryBlock;
    const int64_t head_off = bh * P.N * D;
    const char* kbase = static_cast<const char*>(P.k) + head_off * ESZ;
    const char* vbase = static_cast<const char*>(P.v) + head_off * ESZ;

    int64_t base = 0, cnt = P.M;
    if (!DENSE) {
        base = P.rowptr[row];
        cnt = P.rowptr[row + 1] - base;
    }
    const int64_t ntiles = (cnt + kTileBlocks - 1) / kTileBlocks;
    const int cnt32 = static_cast<int>(cnt);              // <= M < 2^19

    // ---- the wave's queries as the B operand of S^T = K Q^T ----
    const int64_t my_q = q0 + wave * 32 + col;
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
    // Wave w fetches tile blocks 4w..4w+3; lane (sub, c) of a pass covers
    // block sub of the pass, K bytes [16c, 16c+16) of the block (key c/(D/8))
    // and V channel pair c of its 4 keys. Block ids and log-weights are
    // wave-uniform (scalar loads).
    const int c = lane % LPB;
    const int sub = lane / LPB;
    const uint32_t k_lane_off = static_cast<uint32_t>(((c / (D / 8)) * D + (c % (D / 8)) * 8) * ESZ);
    TileRegs<D, F32> R;
    // Plan entries of one tile: lane j < 16 holds block id j of the tile and
    // lane 16 + j the bits of its fp32 log-weight: one coalesced load per
    // tile (a single instruction with a per-lane address), fetched a tile
    // ahead of the gather and broadcast to the wave with readlane.
    int iv = 0;
    auto load_plan = [&](int64_t t) {
        if (DENSE) return;
        const int64_t gb = t * kTileBlocks + (lane & 15);
        const int64_t e = base + ((gb < cnt) ? gb : (cnt - 1));
        const int* src = (lane & 16) ? reinterpret_cast<const int*>(P.logw) + e : P.idx + e;
        iv = *src;
    };
    // Gather of one tile into registers; all K loads are issued before the V
    // loads, so that storing K waits only for the K half.
    auto load_tile = [&](int64_t t) {
        const int t32 = static_cast<int>(t);
        uint32_t boff[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            int blk_s[BPP];
            float lw_s[BPP];
#pragma unroll
            for (int j = 0; j < BPP; ++j) {
                const int tb = wave * 4 + p * BPP + j;
                const int gb = t32 * kTileBlocks + tb;
                if (DENSE) {
                    blk_s[j] = (gb < cnt32) ? gb : (cnt32 - 1);
                    lw_s[j] = (gb < cnt32) ? 0.0f : -INFINITY;
                } else {
                    blk_s[j] = __builtin_amdgcn_readlane(iv, tb);
                    const float lw = __int_as_float(__builtin_amdgcn_readlane(iv, 16 + tb));
                    lw_s[j] = (gb < cnt32) ? lw * kLog2e : -INFINITY;
                }
            }
            const int blk = (BPP == 1 || sub == 0) ? blk_s[0] : blk_s[BPP - 1];
            R.lw[p] = (BPP == 1 || sub == 0) ? lw_s[0] : lw_s[BPP - 1];
            boff[p] = static_cast<uint32_t>(blk) * BLOCK_BYTES + k_lane_off;
        }
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const char* kp = kbase + static_cast<uint64_t>(boff[p]);
            if constexpr (F32) {
                R.k[p][0] = *reinterpret_cast<const float4*>(kp);
                R.k[p][1] = *reinterpret_cast<const float4*>(kp + 16);
            } else {
                R.k[p] = *reinterpret_cast<const uint4*>(kp);
            }
        }
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const char* vp = vbase + static_cast<uint64_t>(boff[p]);
            if constexpr (F32) {
                R.v[p][0] = *reinterpret_cast<const float4*>(vp);
                R.v[p][1] = *reinterpret_cast<const float4*>(vp + 16);
            } else {
                R.v[p] = *reinterpret_cast<const uint4*>(vp);
            }
        }
    };
    auto to_bf16x8 = [](const float4& a, const float4& b) {
        return make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                          pack_bf16x2(b.z, b.w));
    };
    auto store_k = [&](int buf) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int tb = wave * 4 + p * BPP + sub;
            const int key = tb * kKvBlock + c / (D / 8);
            const int d0 = (c % (D / 8)) * 8;
            uint4 ku;
            if constexpr (F32) ku = to_bf16x8(R.k[p][0], R.k[p][1]);
            else ku = R.k[p];
            *reinterpret_cast<uint4*>(&Ks[buf][key * KS + d0]) = ku;
        }
    };
    auto store_v = [&](int buf) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int tb = wave * 4 + p * BPP + sub;
            const int key = tb * kKvBlock + c / (D / 8);
            const int d0 = (c % (D / 8)) * 8;
            uint4 vu;
            if constexpr (F32) vu = to_bf16x8(R.v[p][0], R.v[p][1]);
            else vu = R.v[p];
            const int vchunk = (d0 >> 3) ^ (vseg_swizzle<D>(key) << 2);
            *reinterpret_cast<uint4*>(&Vs[buf][key * D + vchunk * 8]) = vu;
            if (c == 0) lws[buf][tb] = R.lw[p];
        }
    };

    // Transpose-read addressing of the A operand of O^T = V^T P^T: lane
    // (group g = lane/16, rho = lane%16) supplies key row
    // 16*slice + 4*(g/2) + rho/4 (+8 for the second half of the operand) and
    // channels 32*j + 16*(g%2) + 4*(rho%4) .. +3; it receives channel
    // 32*j + lane%32 of the 4 keys, in the key order of the P accumulators.
    const int trg = lane >> 4, rho = lane & 15;
    const int tr_row = 4 * (trg >> 1) + (rho >> 2);
    const int tr_swz = vseg_swizzle<D>(tr_row);
    auto v_operand = [&](int buf, int j, int slice) {
        const int chunk = ((j * 32 + 16 * (trg & 1) + 4 * (rho & 3)) >> 3) ^ (tr_swz << 2);
        const uint16_t* p0 = &Vs[buf][(slice * 16 + tr_row) * D + chunk * 8 + (rho & 1) * 4];
        const uint2 lo = ds_read_tr16(p0);
        const uint2 hi = ds_read_tr16(p0 + 8 * D);
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
    };

    struct SAcc { floatx16 v[2]; };
    // S^T of one tile (64 keys x the wave's 32 queries).
    auto qk = [&](int buf) {
        SAcc S;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            S.v[kb] = floatx16{};
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const uint4 a = *reinterpret_cast<const uint4*>(
                    &Ks[buf][(kb * 32 + col) * KS + s * 16 + half * 8]);
                S.v[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qb[s], S.v[kb], 0, 0, 0);
            }
        }
        return S;
    };

    floatx16 O[ND];
#pragma unroll
    for (int j = 0; j < ND; ++j) O[j] = floatx16{};
    float m_run = -INFINITY, l_run = 0.0f;
    const float scale = P.scale_log2;

    // Online softmax of one tile as a list of work items that the loop below
    // spreads between MFMAs: 8 group maxima, 1 finalisation (cross-half max,
    // new running max, rescale factor, per-group exponent bias), 32
    // exponentials and 16 bf16 packs of P.
    //
    // Accumulator group g of block kb holds the 4 keys of tile block
    // kb*8 + 2g + half: one log-weight per group. The max over a group's raw
    // products times the scale plus the log-weight is the group's max logit
    // (scale > 0). alpha is 1 exactly when the running max did not grow, and
    // 0 on the first tile (m_run = -inf; a first tile always holds a valid
    // block, so its max is finite).
    constexpr int kSmItems = 8 + 1 + 32 + 16;
    // The running max and the row sum are kept as 4 partials each (items
    // rotate over them) so that their updates form short dependency chains.
    // The row sum adds the bf16-rounded weights (one v_dot2 per packed pair
    // against (1, 1)): numerator and normaliser then use the same weights.
    struct SmState {
        float lwv[2][4];
        float bias[2][4];
        float mx[4], psum[4];
        float alpha;
    };
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t ones2 = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
    auto sm_item = [&](int it, SAcc& S, SmState& st, uint32_t (&pw)[4][4]) {
        if (it < 8) {
            const int kb = it >> 2, g = it & 3;
            const float gm = fmaxf(__builtin_fmaxf(S.v[kb][4 * g], S.v[kb][4 * g + 1]) ,
                                   fmaxf(S.v[kb][4 * g + 2], S.v[kb][4 * g + 3]));
            st.mx[it & 3] = fmaxf(st.mx[it & 3], fmaf(gm, scale, st.lwv[kb][g]));
        } else if (it == 8) {
            const float mx = half_max(fmaxf(fmaxf(st.mx[0], st.mx[1]), fmaxf(st.mx[2], st.mx[3])));
            const float m_new = fmaxf(m_run, mx);
            st.alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int g = 0; g < 4; ++g) st.bias[kb][g] = st.lwv[kb][g] - m_new;
            }
        } else if (it < 41) {
            const int e = it - 9, kb = e >> 4, i = e & 15;
            S.v[kb][i] = __builtin_amdgcn_exp2f(fmaf(S.v[kb][i], scale, st.bias[kb][i >> 2]));
        } else {
            // pw[slice][w] = bf16 pair (2w, 2w+1) of the 8 weights of 16-key
            // slice `slice` held by this lane
            const int k = it - 41, slice = k >> 2, w = k & 3;
            const int kb = slice >> 1, o = (slice & 1) * 8 + 2 * w;
            pw[slice][w] = pack_bf16x2(S.v[kb][o], S.v[kb][o + 1]);
            st.psum[k & 3] = __builtin_amdgcn_fdot2_f32_bf16(
                __builtin_bit_cast(bf16x2_t, pw[slice][w]), ones2, st.psum[k & 3], false);
        }
    };

    // Software pipeline over tiles (one barrier per tile). LDS buffer b holds
    // K and V of tiles b, b+2, ...; iteration t runs tile t+1's S^T MFMAs
    // alongside tile t's softmax, then tile t's P V MFMAs. K of tile t+2
    // goes into the K half of buffer t%2 (free since tile t's S^T ran in
    // iteration t-1) before the barrier, V of tile t+2 into the V half after
    // it; the loads for tile t+3 are then issued.
    if (ntiles > 0) { load_plan(0); load_tile(0); store_k(0); store_v(0); }
    if (ntiles > 1) { load_plan(1); load_tile(1); store_k(1); store_v(1); }
    __syncthreads();
    if (ntiles > 2) { load_plan(2); load_tile(2); }
    if (ntiles > 3) load_plan(3);
    // Every wave runs the same instruction stream (a wave whose queries lie
    // past N computes on zero queries and stores nothing), which keeps the
    // loop free of branches around its loads and MFMAs.
    SAcc Sa = qk(0);
    // every wave has read K of tile 0 before iteration 0 overwrites it
    __syncthreads();
    // One pipeline step on tile t: Scur holds S^T of tile t, Snext receives
    // S^T of tile t+1. The loop runs two steps per iteration with the roles
    // of the two accumulator sets swapped, so no registers are copied.
    auto step = [&](int64_t t, SAcc& Scur, SAcc& Snext) {
        const int buf = static_cast<int>(t & 1);
        {
            // Phase A: S^T of tile t+1 (from the other buffer; on the last
            // tile that is stale K and the result is never used), one MFMA
            // per chunk with its K operand read two chunks ahead, and the
            // softmax items of tile t spread over the chunks.
            SmState st;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                st.mx[k] = -INFINITY;
                st.psum[k] = 0.0f;
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int g = 0; g < 4; ++g) st.lwv[kb][g] = lws[buf][kb * 8 + 2 * g + half];
            }
            constexpr int QS = 2 * NS;
            // step i: key half i&1 (the two accumulator chains alternate),
            // channel step i>>1
            auto kread = [&](int i) {
                const int kb = i & 1, s2 = i >> 1;
                return *reinterpret_cast<const uint4*>(
                    &Ks[buf ^ 1][(kb * 32 + col) * KS + s2 * 16 + half * 8]);
            };
            uint4 ka[QS];
            ka[0] = kread(0);
            ka[1] = kread(1);
            SAcc& Sn = Snext;
            Sn.v[0] = floatx16{};
            Sn.v[1] = floatx16{};
            uint32_t pw[4][4];
            // Softmax items of phase A: the group maxima, the finalisation,
            // and the exponentials and packs of keys 0..31 (accumulator kb=0);
            // those of keys 32..63 go to phase B.
            constexpr int kItemsA = 25 + 8, kItemsB = 16 + 8;
            auto item_a = [](int ia) { return ia < 25 ? ia : 41 + (ia - 25); };
            auto item_b = [](int ib) { return ib < 16 ? 25 + ib : 49 + (ib - 16); };
#pragma unroll
            for (int c = 0; c < QS; ++c) {
                if (c + 2 < QS) ka[c + 2] = kread(c + 2);
                Sn.v[c & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    as_bf16x8(ka[c]), qb[c >> 1], Sn.v[c & 1], 0, 0, 0);
#pragma unroll
                for (int ia = c * kItemsA / QS; ia < (c + 1) * kItemsA / QS; ++ia)
                    sm_item(item_a(ia), Scur, st, pw);
                __builtin_amdgcn_sched_barrier(0);
            }
            // Keep the packed weights of keys 0..31 computed here, inside the
            // interleaved phase: without this the compiler sinks them past
            // the rescale branch below, next to their use.
#pragma unroll
            for (int sl = 0; sl < 2; ++sl)
                asm volatile("" : : "v"(pw[sl][0]), "v"(pw[sl][1]), "v"(pw[sl][2]), "v"(pw[sl][3]));
            // The output is rescaled only in tiles where some lane's running
            // max grew (alpha < 1 there; exactly 1 elsewhere).
            if (__builtin_amdgcn_ballot_w64(st.alpha != 1.0f) != 0) {
#pragma unroll
                for (int j = 0; j < ND; ++j) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) O[j][i] *= st.alpha;
                }
            }
            // Phase B: P V, one MFMA per chunk with the V^T operands read two
            // chunks ahead: first the two 16-key slices of keys 0..31 (for
            // every output block) next to the softmax items of keys 32..63,
            // then the slices of keys 32..63.
            constexpr int PS = 4 * ND;
            constexpr int PHALF = 2 * ND;
            auto pv_at = [](int c) { return c < PHALF ? (c / ND) : 2 + (c - PHALF) / ND; };
            uint4 va[PS];
            va[0] = v_operand(buf, 0 % ND, pv_at(0));
            va[1] = v_operand(buf, 1 % ND, pv_at(1));
#pragma unroll
            for (int c = 0; c < PS; ++c) {
                if (c + 2 < PS) va[c + 2] = v_operand(buf, (c + 2) % ND, pv_at(c + 2));
                const int j = c % ND, sl = pv_at(c);
                O[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    as_bf16x8(va[c]), as_bf16x8(make_uint4(pw[sl][0], pw[sl][1], pw[sl][2], pw[sl][3])),
                    O[j], 0, 0, 0);
                if (c < PHALF) {
#pragma unroll
                    for (int ib = c * kItemsB / PHALF; ib < (c + 1) * kItemsB / PHALF; ++ib)
                        sm_item(item_b(ib), Scur, st, pw);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            l_run = fmaf(l_run, st.alpha, (st.psum[0] + st.psum[1]) + (st.psum[2] + st.psum[3]));
            // K of tile t+2, as late as the barrier allows (unconditional:
            // past the row's end it writes stale K that only the discarded
            // S^T of the last tile reads)
            store_k(buf);
        }
        __syncthreads();
        // V of tile t+2 (past the row's end: stale data nobody reads)
        store_v(buf);
        if (t + 3 < ntiles) load_tile(t + 3);
        if (t + 4 < ntiles) load_plan(t + 4);
    };
    SAcc Sb;
    for (int64_t t = 0; t < ntiles; t += 2) {
        step(t, Sa, Sb);
        if (t + 1 < ntiles) step(t + 1, Sb, Sa);
    }

    const float l_tot = half_sum(l_run);
    if (my_q >= P.N) return;
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
