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
// wave w owns queries [32w, 32w+32); the dense comparator takes two
// neighbouring rows of a head per workgroup of 8 waves, sharing their tiles):
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
//     LDS buffers hold K, V and log-weights of alternate tiles. The gather
//     goes straight from global memory into LDS (global_load_lds_dwordx4,
//     16 bytes per lane, no registers and no LDS store instructions): at the
//     start of iteration t the waves issue K of tile t+2 and V of tile t+1
//     into the buffers that iteration t-1 finished reading; each wave waits
//     for its loads before the barrier that ends iteration t, which
//     publishes them.
//     Each lane picks the global address of the 16 bytes its LDS slot must
//     hold, which is how the bank swizzles of both tiles are applied. Two
//     workgroups per CU. Block ids come from one plan load per tile,
//     broadcast with readlane; gather addresses are 32-bit offsets from the
//     head's base.
//   * fp32 inputs are rounded to bf16 by a separate pass before the kernel
//     (round to nearest even, the rounding the products use either way).
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

#include <mutex>
#include <type_traits>
#include <vector>

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
template <int D> __device__ __forceinline__ constexpr int vseg_swizzle(int key) {
    return (D == 128) ? (key & 3) : ((key >> 1) & 1);
}

// K tiles are stored row-major [key][channel] without padding; 16-byte
// column c of key row `key` sits at column c ^ kcol_swizzle(key), so that the
// K operand reads (one column of 16 consecutive keys per 16 lanes) hit
// distinct LDS banks.
template <int D> __device__ __forceinline__ constexpr int kcol_swizzle(int key) {
    return (D == 128) ? (key & 15) : ((key >> 1) & 7);
}

typedef __attribute__((address_space(3))) void lds_void;
template <int V> using IntC = std::integral_constant<int, V>;

// 16 bytes per lane from base + off straight into LDS: lane l's bytes land
// at lds_dst + 16 l (global_load_lds_dwordx4, LDS base in M0). Written as
// inline asm so that the compiler does not order every later LDS read of
// the workgroup behind it; the loads complete under the kernel's own
// s_waitcnt vmcnt(0) before the barrier that publishes them. The s_nop
// gives the 5 wait states the load needs after a VALU write of its base
// SGPRs (the compiler may restore spilled SGPRs with v_readlane right
// before the asm, and does not check hazards inside it); it also covers
// the one after the M0 write.
__device__ __forceinline__ void load_to_lds(const char* base, uint32_t off, uint16_t* lds_dst) {
    const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)lds_dst));
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(m0)
                 : "memory");
}
__device__ __forceinline__ void wait_lds_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Rows per workgroup: the dense comparator runs two neighbouring query blocks
// of a head in one workgroup of 8 waves, which need the same K/V tiles, so
// each tile is gathered once for both (half the gather and HBM traffic per
// query); every wave's own work is unchanged, so its output is the same bit
// for bit. A sparse row has its own blocks: one row of 4 waves.
template <bool DENSE> constexpr int kRowsPerGroup = DENSE ? 2 : 1;

template <int D, bool OUT_F32, bool DENSE>
__global__ __launch_bounds__(256 * kRowsPerGroup<DENSE>, 2 / kRowsPerGroup<DENSE>) void attn_kernel(
    AttnParams P) {
    constexpr int RW = kRowsPerGroup<DENSE>;
    constexpr int NW = 4 * RW;                  // waves per workgroup
    constexpr int NS = D / 16;                  // 16-channel MFMA steps
    constexpr int ND = D / 32;                  // 32-channel output blocks
    constexpr int ROWB = D * 2;                 // bytes of one bf16 key row
    constexpr uint32_t BLOCK_BYTES = kKvBlock * ROWB;
    constexpr int CPW = kTileKeys * ROWB / 1024 / NW;  // 1 KB gather chunks per wave
    static_assert(CPW >= 1, "every wave gathers at least one chunk");
    constexpr int KPC = 1024 / ROWB;            // key rows per chunk
    // the two K buffers are one array, so a K operand address is one
    // loop-invariant register plus an immediate offset for buffer and key half
    __shared__ __align__(16) uint16_t Ks[2][kTileKeys * D];
    __shared__ __align__(16) uint16_t Vs0[kTileKeys * D], Vs1[kTileKeys * D];
    __shared__ float lws0[kTileBlocks], lws1[kTileBlocks];
    // Buffer b of each kind; b is a compile-time constant at every use.
    auto Kbuf = [&](auto b) -> uint16_t* { return Ks[decltype(b)::value]; };
    auto Vbuf = [&](auto b) -> uint16_t* { if constexpr (decltype(b)::value) return Vs1; else return Vs0; };
    auto Lbuf = [&](auto b) -> float* { if constexpr (decltype(b)::value) return lws1; else return lws0; };

    // Work unit = RW consecutive query blocks of one head (a row, or a pair
    // of rows; with an odd QB the last pair has one real row and the second
    // half computes on no queries).
    const int bid = blockIdx.x;
    const int64_t unit = static_cast<int64_t>(bid % kXcds) * P.per_xcd + bid / kXcds;
    const int64_t units_per_head = (P.QB + RW - 1) / RW;
    if (unit >= P.rows / P.QB * units_per_head) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int half = lane >> 5;

    const int64_t bh = unit / units_per_head;
    const int64_t r = (unit - bh * units_per_head) * RW + wave / 4;   // this wave's query block
    const int64_t row = bh * P.QB + r;          // its plan row (sparse: RW = 1, r < QB)
    const int64_t q0 = r * kQueryBlock;
    const int64_t head_off = bh * P.N * D;
    const char* kbase = static_cast<const char*>(P.k) + head_off * 2;
    const char* vbase = static_cast<const char*>(P.v) + head_off * 2;

    int64_t base = 0, cnt = P.M;
    if (!DENSE) {
        base = P.rowptr[row];
        cnt = P.rowptr[row + 1] - base;
    }
    const int cnt32 = static_cast<int>(cnt);              // <= M < 2^19
    const int ntiles = (cnt32 + kTileBlocks - 1) / kTileBlocks;

    // ---- the wave's queries as the B operand of S^T = K Q^T ----
    const int64_t my_q = q0 + (wave & 3) * 32 + col;
    bf16x8 qb[NS];
    {
        const bool ok = my_q < P.N;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int dd = s * 16 + half * 8;
            uint4 u = make_uint4(0, 0, 0, 0);
            if (ok)
                u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(P.q) + head_off +
                                                    my_q * D + dd);
            qb[s] = as_bf16x8(u);
        }
    }

    // Plan entries of one tile: lane j < 16 holds block id j of the tile and
    // lane 16 + j the bits of its fp32 log-weight (one coalesced load per
    // tile; entries past the row's end repeat its last entry).
    const int* plan_src = DENSE ? nullptr
                                : ((lane & 16) ? reinterpret_cast<const int*>(P.logw) : P.idx) + base;
    auto load_plan = [&](int t) -> int {
        if (DENSE) return 0;
        const int gb = t * kTileBlocks + (lane & 15);
        return plan_src[(gb < cnt32) ? gb : (cnt32 - 1)];
    };
    // Direct gather of K or V of tile T into buffer b. Wave w fills the 1 KB
    // LDS chunks w*CPW .. w*CPW+CPW-1 of the tile; lane l's 16 bytes land at
    // byte 16 l of its chunk, i.e. key row lkey, stored column lcol, and the
    // lane loads the logical column that the swizzle puts there.
    const int lkey = lane / (ROWB / 16);
    const int lcol = lane % (ROWB / 16);
    // With one block per chunk (d = 128) a chunk's block address goes into
    // the load's scalar base (scalar arithmetic) and each lane adds a fixed
    // offset: that of its key row within the block and its swizzled column.
    // The offsets depend on the chunk only through i (the wave's chunks
    // start at a multiple of 16 keys, the swizzle period), so they are
    // computed once.
    uint32_t goff[2][CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const int key = (wave * CPW + i) * KPC + lkey;
        goff[0][i] = static_cast<uint32_t>((key & 3) * ROWB + (lcol ^ kcol_swizzle<D>(key)) * 16);
        goff[1][i] = static_cast<uint32_t>((key & 3) * ROWB + (lcol ^ (vseg_swizzle<D>(key) << 2)) * 16);
        if constexpr (KPC == 4 && !DENSE) asm volatile("" : "+v"(goff[0][i]), "+v"(goff[1][i]));
    }
    auto gather = [&](auto is_v, auto b, int ivt, int T32) {
        constexpr bool ISV = decltype(is_v)::value;
        const char* gsrc = ISV ? vbase : kbase;
        uint16_t* dst = ISV ? Vbuf(b) : Kbuf(b);
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int ch = wave * CPW + i;
            if constexpr (KPC == 4 && !DENSE) {
                const uint32_t blk = static_cast<uint32_t>(__builtin_amdgcn_readlane(ivt, ch));
                load_to_lds(gsrc + blk * BLOCK_BYTES, goff[ISV][i], dst + ch * 512);
                continue;
            }
            const int key = ch * KPC + lkey;                // key of the tile, 0..63
            int blk;
            if (DENSE) {
                const int gb = T32 * kTileBlocks + (key >> 2);
                blk = (gb < cnt32) ? gb : (cnt32 - 1);
            } else {
                const int b0 = __builtin_amdgcn_readlane(ivt, 2 * ch);
                const int b1 = __builtin_amdgcn_readlane(ivt, 2 * ch + 1);
                blk = (lkey >= 4) ? b1 : b0;
            }
            const int lc = ISV ? (lcol ^ (vseg_swizzle<D>(key) << 2)) : (lcol ^ kcol_swizzle<D>(key));
            const uint32_t off = static_cast<uint32_t>(blk) * BLOCK_BYTES +
                                 static_cast<uint32_t>((key & 3) * ROWB + lc * 16);
            load_to_lds(gsrc, off, dst + ch * 512);
        }
    };
    // Log-weights of tile T (log2 units; -inf past the row's end) into buffer b.
    auto write_lws = [&](auto b, int ivt, int T) {
        if (wave == 0 && (lane >> 4) == 1) {
            const int j = lane - 16;
            const bool ok = T * kTileBlocks + j < cnt32;
            const float lw = DENSE ? 0.0f : __int_as_float(ivt) * kLog2e;
            Lbuf(b)[j] = ok ? lw : -INFINITY;
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
    auto v_operand = [&](auto b, int j, int slice) {
        const int chunk = ((j * 32 + 16 * (trg & 1) + 4 * (rho & 3)) >> 3) ^ (tr_swz << 2);
        const uint16_t* p0 = Vbuf(b) + (slice * 16 + tr_row) * D + chunk * 8 + (rho & 1) * 4;
        const uint2 lo = ds_read_tr16(p0);
        const uint2 hi = ds_read_tr16(p0 + 8 * D);
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
    };

    // K operand of MFMA step s2 for key half kb: key row kb*32 + col,
    // logical 16-byte column 2*s2 + half. Rows col and 32 + col have the
    // same swizzle, so the key half is an offset of 32 rows; the byte offset
    // of each step is computed once.
    static_assert(kcol_swizzle<D>(0) == kcol_swizzle<D>(32) && kcol_swizzle<D>(5) == kcol_swizzle<D>(37),
                  "K swizzle period must divide 32 rows");
    uint32_t koff[NS];
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) {
        koff[s2] = static_cast<uint32_t>(col * ROWB + (((2 * s2 + half) ^ kcol_swizzle<D>(col)) * 16));
        asm volatile("" : "+v"(koff[s2]));
    }
    auto k_operand = [&](auto b, int kb, int s2) {
        const char* p = reinterpret_cast<const char*>(Kbuf(b)) + kb * 32 * ROWB;
        return *reinterpret_cast<const uint4*>(p + koff[s2]);
    };

    struct SAcc { floatx16 v[2]; };
    // S^T of one tile (64 keys x the wave's 32 queries).
    auto qk = [&](auto b) {
        SAcc S;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            S.v[kb] = floatx16{};
#pragma unroll
            for (int s = 0; s < NS; ++s)
                S.v[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(k_operand(b, kb, s)),
                                                                  qb[s], S.v[kb], 0, 0, 0);
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

    // Software pipeline over tiles (one barrier per tile). Buffer b holds K,
    // V and log-weights of tiles b, b+2, ...; iteration t runs tile t+1's
    // S^T MFMAs alongside tile t's softmax, then tile t's P V MFMAs. It
    // first issues the gathers of K of tile t+2 (into buffer t%2, whose K
    // was read by the S^T MFMAs of iteration t-1) and of V and log-weights of
    // tile t+1 (into buffer (t+1)%2, read in iteration t-1), and the plan
    // entries of tile t+3.
    int iv1 = 0, iv2 = 0;
    {
        const int iv0 = (ntiles > 0) ? load_plan(0) : 0;
        iv1 = (ntiles > 1) ? load_plan(1) : 0;
        iv2 = (ntiles > 2) ? load_plan(2) : 0;
        if (ntiles > 0) {
            gather(IntC<0>{}, IntC<0>{}, iv0, 0);
            gather(IntC<1>{}, IntC<0>{}, iv0, 0);
            write_lws(IntC<0>{}, iv0, 0);
        }
        if (ntiles > 1) gather(IntC<0>{}, IntC<1>{}, iv1, 1);
    }
    wait_lds_loads();
    __syncthreads();
    // Every wave runs the same instruction stream (a wave whose queries lie
    // past N computes on zero queries and stores nothing), which keeps the
    // loop free of branches around its loads and MFMAs.
    SAcc Sa = qk(IntC<0>{});
    // every wave has read K of tile 0 before iteration 0 overwrites it
    __syncthreads();
    // One pipeline step on tile t (buffer b = t % 2): Scur holds S^T of tile
    // t, Snext receives S^T of tile t+1. The loop runs two steps per
    // iteration with the roles of the two accumulator sets swapped, so no
    // registers are copied.
    auto step = [&](auto b, int t, SAcc& Scur, SAcc& Snext) {
        constexpr int buf = decltype(b)::value;
        const IntC<buf ^ 1> nb{};
        if (t + 2 < ntiles) gather(IntC<0>{}, b, iv2, t + 2);
        if (t + 1 < ntiles) {
            gather(IntC<1>{}, nb, iv1, t + 1);
            write_lws(nb, iv1, t + 1);
        }
        const int ivn = (t + 3 < ntiles) ? load_plan(t + 3) : 0;
        {
            // Phase A: S^T of tile t+1 (from the other buffer; on the last
            // tile that is stale K and the result is never used), one MFMA
            // per chunk with its K operand read two chunks ahead, and the
            // softmax items of tile t spread over the chunks.
            // A wave runs its QK^T phase at raised priority, so that while
            // it streams these MFMAs the other wave of the SIMD, in its VALU
            // heavy P V phase, fills the issue slots in between (measured:
            // about 1.3% faster; raising it over the P V phase instead gained
            // nothing).
            __builtin_amdgcn_s_setprio(1);
            SmState st;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                st.mx[k] = -INFINITY;
                st.psum[k] = 0.0f;
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int g = 0; g < 4; ++g) st.lwv[kb][g] = Lbuf(b)[kb * 8 + 2 * g + half];
            }
            constexpr int QS = 2 * NS;
            // step i: key half i&1 (the two accumulator chains alternate),
            // channel step i>>1
            auto kread = [&](int i) { return k_operand(nb, i & 1, i >> 1); };
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
            __builtin_amdgcn_s_setprio(0);
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
            va[0] = v_operand(b, 0 % ND, pv_at(0));
            va[1] = v_operand(b, 1 % ND, pv_at(1));
#pragma unroll
            for (int c = 0; c < PS; ++c) {
                if (c + 2 < PS) va[c + 2] = v_operand(b, (c + 2) % ND, pv_at(c + 2));
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
        }
        // This wave's gathers are complete; after the barrier every wave's
        // gathers of this iteration are visible.
        wait_lds_loads();
        __syncthreads();
        iv1 = iv2;
        iv2 = ivn;
    };
    SAcc Sb;
    for (int t = 0; t < ntiles; t += 2) {
        step(IntC<0>{}, t, Sa, Sb);
        if (t + 1 < ntiles) step(IntC<1>{}, t + 1, Sb, Sa);
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
            if constexpr (OUT_F32) {
                float* dst = static_cast<float*>(P.o) + head_off + my_q * D + dd;
                *reinterpret_cast<float4*>(dst) = make_float4(x0, x1, x2, x3);
            } else {
                uint16_t* dst = static_cast<uint16_t*>(P.o) + head_off + my_q * D + dd;
                *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
            }
        }
    }
}

template <int D, bool OUT_F32, bool DENSE>
void launch_one(const AttnParams& p, hipStream_t s) {
    constexpr int RW = kRowsPerGroup<DENSE>;
    const int64_t units = p.rows / p.QB * ((p.QB + RW - 1) / RW);
    AttnParams q = p;
    q.per_xcd = (units + kXcds - 1) / kXcds;
    const int64_t grid = q.per_xcd * kXcds;
    hipLaunchKernelGGL((attn_kernel<D, OUT_F32, DENSE>), dim3(static_cast<unsigned>(grid)),
                       dim3(256 * RW), 0, s, q);
}

// fp32 -> bf16, round to nearest even; 8 elements per thread and iteration.
__global__ __launch_bounds__(256) void to_bf16_kernel(const float* __restrict__ src,
                                                      uint16_t* __restrict__ dst, int64_t n8) {
    for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n8; i += static_cast<int64_t>(gridDim.x) * 256) {
        const float4 a = reinterpret_cast<const float4*>(src)[2 * i];
        const float4 b = reinterpret_cast<const float4*>(src)[2 * i + 1];
        reinterpret_cast<uint4*>(dst)[i] = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w),
                                                      pack_bf16x2(b.x, b.y), pack_bf16x2(b.z, b.w));
    }
}

// Scratch of the allocation-free attention call (bf16 copies of fp32 q, k,
// v): one copy of this array lives on every device the library runs on, for
// the life of the process. Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol); it passes the
// device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint16_t scratch[3 * kNoAllocMaxElems];

std::mutex g_scratch_mutex;
std::vector<uint16_t*> g_scratch_addr;   // per device, null until looked up

}  // namespace

hipError_t noalloc_scratch(uint16_t** out) {
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (static_cast<size_t>(dev) >= g_scratch_addr.size()) g_scratch_addr.resize(dev + 1, nullptr);
    if (!g_scratch_addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_addr[dev] = static_cast<uint16_t*>(p);
    }
    *out = g_scratch_addr[dev];
    return hipSuccess;
}

hipError_t launch_to_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s) {
    const int64_t n8 = n / 8;                   // n is a multiple of 8 (d in {64, 128})
    if (n8 == 0) return hipSuccess;
    int64_t blocks = (n8 + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(to_bf16_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, src,
                       dst, n8);
    return hipGetLastError();
}

hipError_t launch_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, void* o,
                            bool out_f32, int64_t B, int64_t H, int64_t N, int d,
                            const int64_t* rowptr, const int32_t* idx, const float* logw,
                            bool dense, hipStream_t s) {
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
    if (d == 128) {
        if (out_f32) dense ? launch_one<128, true, true>(p, s) : launch_one<128, true, false>(p, s);
        else dense ? launch_one<128, false, true>(p, s) : launch_one<128, false, false>(p, s);
    } else {
        if (out_f32) dense ? launch_one<64, true, true>(p, s) : launch_one<64, true, false>(p, s);
        else dense ? launch_one<64, false, true>(p, s) : launch_one<64, false, false>(p, s);
    }
    return hipGetLastError();
}

}  // namespace absa
