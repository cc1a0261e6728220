// SSD chunked-scan forward kernels for gfx950 (MI355X).
//
// Two kernels make one forward pass:
//
//  1. ssd_prep_kernel, one workgroup per (row, group, block of QB tokens):
//       CB[t][s] = C_t . B_s   for t, s in the block (fp32), and B^T of the block.
//     These depend only on B and C, so every head of the group reuses them;
//     they are the intra-chunk C B^T products of the dual form Y = [L o (C B^T)] X
//     ("088 Mamba-2", section 2.2; the diagonal-block step of key design 2 on
//     the "Mamba-2 - Transformer and SSM share one algebra" page).
//
//  2. ssd_scan_kernel, one workgroup per (row, head), P/16 waves; wave w owns
//     channels p in [16w, 16w+16).  The workgroup walks its row block by block
//     (QB = 32 or 64 tokens) with the P x N state held in MFMA accumulator
//     registers for the whole row.  Per block:
//       a. log-decay l_t = dt_t A_h (kept in log2 units) and its inclusive
//          cumulative sum within the block, by a wavefront scan
//          (the within-chunk cumsum of the chunked algorithm);
//       b. masked decay L[t][s] = exp(cum_t - cum_s) for s <= t in the same
//          sequence, else 0, multiplied into CB (segment sum, section 2.2);
//       c. y_diag = (L o CB) X on bf16 MFMA (diagonal block, section 2.3);
//       d. y_off  = exp(cum_t) C_t H_prev, the incoming state read out by C and
//          decayed to each position (left factor, section 3 of "088 Mamba-2");
//       e. H <- exp(cum_end) H + X^T (exp(cum_end - cum_s) o B), the block's end
//          state combined with the carried one (right factor and the
//          inter-chunk scan step real_end = block_decay * prev + local_end);
//       f. y = y_off + y_diag + D x, written once to HBM in fp32.
//     Sequence boundaries inside a block (seq_idx) split it into segments:
//     L is masked across segments, each segment's incoming state is either the
//     carried state or its own initial state, and the state of a sequence that
//     ends inside the block is written to final_state on the spot.
//
// Because the state stays in registers, x is read once and y written once;
// the only other traffic is dt and the per-block CB / B^T tiles, which all
// heads of a group share through L2.

#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- MFMA traits
// 16x16 output tiles.  Accumulator layout (both types): lane l holds rows
// 4*(l/16) + i, i = 0..3, of column l % 16.  Operand layout: lane l holds row
// (A) or column (B) l % 16 and K values KPL*(l/16) .. KPL*(l/16)+KPL-1 of the
// KSTEP-wide step.
template <typename TI> struct Mfma;
template <> struct Mfma<__bf16> {
    static constexpr int KPL = 8, KSTEP = 32;
    typedef bf16x8 frag;
    __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<float> {
    static constexpr int KPL = 1, KSTEP = 4;
    typedef float frag;
    __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

template <typename TI> __device__ inline TI to_in(float v);
template <> __device__ inline __bf16 to_in<__bf16>(float v) { return (__bf16)v; }
template <> __device__ inline float to_in<float>(float v) { return v; }
__device__ inline float to_f32(__bf16 v) { return (float)v; }
__device__ inline float to_f32(float v) { return v; }

// K-contiguous fragment from LDS (16-byte aligned for bf16).
template <typename TI> __device__ inline typename Mfma<TI>::frag lds_frag(const TI* p);
template <> __device__ inline bf16x8 lds_frag<__bf16>(const __bf16* p) { return *(const bf16x8*)p; }
template <> __device__ inline float lds_frag<float>(const float* p) { return *p; }

__device__ inline float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }

// Rows of the state tiles.  The state S (P x N) is held transposed, S^T[n][p],
// as N/16 accumulator tiles per wave; accumulator row rho = 4*(l/16) + i of
// tile m holds state row n = nrow(m, rho).  For N % 32 == 0 the rows of tile
// pairs (2k, 2k+1) are interleaved so that lane group l/16 of the pair holds
// the 8 consecutive rows 32k + 8*(l/16) .. +7: converted to bf16 they are
// exactly the B operand of the read-out C . S^T for the K step k, and the A
// operand (C) is one contiguous 16-byte read.  The permutation is applied to
// the rows of the B^T operand that produces the state, so no data moves.
template <int N>
__device__ inline int nrow(int m, int rho) {
    if constexpr (N % 32 == 0) return 32 * (m >> 1) + 8 * (rho >> 2) + 4 * (m & 1) + (rho & 3);
    else return 16 * m + rho;
}

// K steps of the read-out product C . S^T (K = N).
template <typename TI, int N> struct OffK {
    static constexpr int NK = N / Mfma<TI>::KSTEP;
};

// B-operand fragments of the read-out from the state accumulators.
template <int N>
__device__ inline void state_frags(const f32x4 (&st)[N / 16], bf16x8 (&sf)[N / 32]) {
#pragma unroll
    for (int k = 0; k < N / 32; ++k) {
        bf16x8 f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[i] = (__bf16)st[2 * k][i];
            f[4 + i] = (__bf16)st[2 * k + 1][i];
        }
        sf[k] = f;
    }
}
template <int N>
__device__ inline void state_frags(const f32x4 (&st)[N / 16], float (&sf)[N / 4]) {
#pragma unroll
    for (int m = 0; m < N / 16; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) sf[4 * m + i] = st[m][i];
}

// Same fragments from an fp32 state row in global memory (row p = this lane's channel).
template <int N>
__device__ inline void global_state_frags(const float* row, int lg, bf16x8 (&sf)[N / 32]) {
#pragma unroll
    for (int k = 0; k < N / 32; ++k) {
        const float4 lo = *(const float4*)(row + 32 * k + 8 * lg);
        const float4 hi = *(const float4*)(row + 32 * k + 8 * lg + 4);
        bf16x8 f;
        f[0] = (__bf16)lo.x; f[1] = (__bf16)lo.y; f[2] = (__bf16)lo.z; f[3] = (__bf16)lo.w;
        f[4] = (__bf16)hi.x; f[5] = (__bf16)hi.y; f[6] = (__bf16)hi.z; f[7] = (__bf16)hi.w;
        sf[k] = f;
    }
}
template <int N>
__device__ inline void global_state_frags(const float* row, int lg, float (&sf)[N / 4]) {
#pragma unroll
    for (int m = 0; m < N / 16; ++m) {
        const float4 v = *(const float4*)(row + nrow<N>(m, 4 * lg));
        sf[4 * m + 0] = v.x; sf[4 * m + 1] = v.y; sf[4 * m + 2] = v.z; sf[4 * m + 3] = v.w;
    }
}

// A-operand fragment of the read-out: row t of the C tile at the K indices of step k.
template <int N>
__device__ inline bf16x8 c_frag(const __bf16* row, int k, int lg) { return *(const bf16x8*)(row + 32 * k + 8 * lg); }
template <int N>
__device__ inline float c_frag(const float* row, int k, int lg) { return row[nrow<N>(k >> 2, 4 * lg + (k & 3))]; }

// Operand fragment of X^T (row = channel p0 + l%16, K = tokens ks + KPL*(l/16) ..)
// read from a row-major tile sX[t][p] (pitch lp elements).  bf16: the LDS
// transpose read; within each group of 16 lanes, lane j reads 4 channels
// p0 + 4(j%4) .. of token row R + j/4, and the hardware hands lane i channel
// p0 + i of rows R .. R+3; two reads give the 8 tokens of one K step.
// fp32: one value per lane, no transpose needed.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ inline bf16x8 x_frag(const __bf16* sX, int lp, int ks, int p0, int lr, int lg) {
    const __bf16* a = sX + (ks + 8 * lg + (lr >> 2)) * lp + p0 + 4 * (lr & 3);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(a + 4 * lp));
    const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo), h4 = __builtin_bit_cast(bf16x4, hi);
    return __builtin_shufflevector(l4, h4, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ inline float x_frag(const float* sX, int lp, int ks, int p0, int lr, int lg) {
    return sX[(ks + lg) * lp + p0 + lr];
}

// Make this wave's LDS writes visible to its own other lanes.
__device__ inline void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Workgroup barrier that orders LDS only.  __syncthreads() also fences global
// memory, which makes every wave wait for all of its outstanding global loads
// (the prefetches of the next blocks) at each barrier; the tiles exchanged
// through barriers here all live in LDS.
__device__ inline void block_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Raw buffer resources: loads outside [0, bytes) return zero and stores there
// are dropped by the hardware range check, so the ragged last block needs no
// per-element guards (and no divergent branches around memory operations).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ inline rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int64_t lim = bytes < 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffffLL : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)lim, 0x00020000);
}
__device__ inline uint4 buf_load16(rsrc_t r, int off) {
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const u4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline uint2 buf_load8(rsrc_t r, int off) {
    typedef unsigned int u2 __attribute__((ext_vector_type(2)));
    const u2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return make_uint2(v.x, v.y);
}
__device__ inline float buf_load_f32(rsrc_t r, int off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ inline int buf_load_i32(rsrc_t r, int off) {
    return __builtin_bit_cast(int, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ inline void buf_store16(f32x4 v, rsrc_t r, int off) {
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, off, 0, 0);
}

struct PrepParams {
    const void* B;
    const void* C;
    float* cb;          // (b, G, nblk, QB, QB) fp32
    void* bt;           // (b, G, nblk, N, QB) input dtype
    int64_t T, G;
    int nblk;
};

struct ScanParams {
    const void* x;
    const float* dt;
    const float* A_log;
    const float* D;
    const float* init;
    const int32_t* seq_idx;
    float* y;
    float* fin;
    const float* cb;
    const void* bt;
    const void* C;
    int64_t batch, T, H, G, nseqs;
    int nblk;
    int dt_scales_x;
};

// ============================================================== prep kernel
template <typename TI, int N, int QB>
__global__ __launch_bounds__(256) void ssd_prep_kernel(PrepParams prm) {
    constexpr int VE = 16 / sizeof(TI);         // elements per 16-byte vector
    constexpr int LP = N + VE;                  // padded row pitch (elements)
    __shared__ __attribute__((aligned(16))) TI sB[QB * LP];
    __shared__ __attribute__((aligned(16))) TI sC[QB * LP];

    const int tid = threadIdx.x;
    const int blk = blockIdx.x % prm.nblk;
    const int64_t bg = blockIdx.x / prm.nblk;   // b * G + g
    const int64_t b = bg / prm.G, g = bg % prm.G;
    const int64_t t0 = (int64_t)blk * QB;
    const int rows = (int)min((int64_t)QB, prm.T - t0);

    const TI* Bg = (const TI*)prm.B;
    const TI* Cg = (const TI*)prm.C;
    for (int v = tid; v < QB * N / VE; v += 256) {
        const int t = v / (N / VE), c = v % (N / VE);
        uint4 bv = make_uint4(0, 0, 0, 0), cv = make_uint4(0, 0, 0, 0);
        if (t < rows) {
            const int64_t off = ((b * prm.T + t0 + t) * prm.G + g) * N + c * VE;
            bv = *(const uint4*)(Bg + off);
            cv = *(const uint4*)(Cg + off);
        }
        *(uint4*)(sB + t * LP + c * VE) = bv;
        *(uint4*)(sC + t * LP + c * VE) = cv;
    }
    __syncthreads();

    // CB = C B^T over the block, 4x4 outputs per thread.
    constexpr int G4 = QB / 4;
    if (tid < G4 * G4) {
        const int tg = tid / G4, sg = tid % G4;
        float acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
        for (int n = 0; n < N; ++n) {
            float cv[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                cv[i] = to_f32(sC[(4 * tg + i) * LP + n]);
                bv[i] = to_f32(sB[(4 * sg + i) * LP + n]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(cv[i], bv[j], acc[i][j]);
        }
        float* out = prm.cb + ((bg * prm.nblk + blk) * QB) * QB;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *(float4*)(out + (4 * tg + i) * QB + 4 * sg) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
    }
    // B^T of the block (rows n, columns s), in the input dtype.
    TI* bt = (TI*)prm.bt + ((bg * prm.nblk + blk) * N) * QB;
    for (int v = tid; v < N * QB; v += 256) {
        const int n = v / QB, s = v % QB;
        bt[v] = sB[s * LP + n];
    }
}

// ============================================================== scan kernel
template <typename TI> struct CumType { typedef float type; };
template <> struct CumType<float> { typedef double type; };   // fp32 path: exponent differences in fp64

// Inclusive prefix sum over the 64 lanes of a wavefront: Hillis-Steele steps
// inside each row of 16 lanes (DPP row shifts), then the row totals are
// broadcast into the following rows.
template <int CTRL, int RMASK>
__device__ inline float dpp_add(float x) {
    const int t = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, RMASK, 0xf, true);
    return x + __builtin_bit_cast(float, t);
}
__device__ inline float wave_incl_scan(float x) {
    x = dpp_add<0x111, 0xf>(x);   // row_shr:1
    x = dpp_add<0x112, 0xf>(x);   // row_shr:2
    x = dpp_add<0x114, 0xf>(x);   // row_shr:4
    x = dpp_add<0x118, 0xf>(x);   // row_shr:8
    x = dpp_add<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
    x = dpp_add<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
    return x;
}
__device__ inline double wave_incl_scan(double x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const double o = __shfl_up(x, d);
        if (lane >= d) x += o;
    }
    return x;
}

template <typename TI, int P, int N, int QB>
struct ScanCfg {
    static constexpr int NW = P / 16;                 // waves; wave w owns channels 16w .. 16w+15
    static constexpr int NT = NW * 64;
    static constexpr int SZ = (int)sizeof(TI);
    static constexpr int VE = 16 / SZ;                // elements per 16-byte vector
    static constexpr int LC = N + VE;                 // pitch of C rows (elements)
    static constexpr int LQ = QB + VE;                // pitch of rows indexed by token s
    static constexpr int LR = P + 32 / SZ;            // pitch of the row-major X tiles (32 bytes of pad:
                                                      // the four rows of a transposed read fall in
                                                      // distinct banks)
    static constexpr int KPL = Mfma<TI>::KPL, KSTEP = Mfma<TI>::KSTEP;
    static constexpr int NK = OffK<TI, N>::NK;
    static constexpr int RT = QB / 16;                // token tiles of a block
    static constexpr int MT = N / 16;                 // state tiles per wave
    static constexpr int NTILE = RT * (RT + 1) / 2;   // causal 16x16 tiles of the decay mask
    // LDS tiles: C, B^T, masked decay L o CB, X and end-state-weighted X (both row-major)
    static constexpr int OFF_C = 0;
    static constexpr int OFF_BT = OFF_C + QB * LC;
    static constexpr int OFF_LM = OFF_BT + N * LQ;
    static constexpr int OFF_XR = OFF_LM + QB * LQ;
    static constexpr int OFF_XW = OFF_XR + QB * LR;
    static constexpr int BUF_ELEMS = OFF_XW + QB * LR;
    // per-thread work units
    static constexpr int CV = QB * N / VE, CPT = (CV + NT - 1) / NT;           // C tile vectors
    static constexpr int BV = N * QB / VE, BPT = (BV + NT - 1) / NT;           // B^T tile vectors
    static constexpr int LMU = NTILE * 64, LMPT = (LMU + NT - 1) / NT;         // 4-element pieces of L o CB
    static constexpr int XC = 8 / SZ;                                          // channels per 8 bytes
    static constexpr int XU = (QB / 4) * (P / XC), XPT = (XU + NT - 1) / NT;   // (4 tokens, XC channels) of X
    // B^T rows n and n + 8 would share LDS banks in the permuted-row reads of
    // the state update; for bf16 64-token blocks the two 64-byte halves of
    // every row with bit 3 of n set are swapped (XOR swizzle, element offset).
    static constexpr bool BT_SWZ = (SZ == 2 && QB == 64);
    __device__ static inline int bt_col(int n, int col) { return BT_SWZ ? (col ^ (((n >> 3) & 1) * 32)) : col; }
};

template <typename TI, int P, int N, int QB, bool SEQ, bool EULER>
__global__ __launch_bounds__(P / 16 * 64) void ssd_scan_kernel(ScanParams prm) {
    typedef ScanCfg<TI, P, N, QB> K;
    typedef Mfma<TI> MF;
    typedef typename MF::frag frag;
    typedef typename CumType<TI>::type cum_t;
    constexpr int NT = K::NT, VE = K::VE, LC = K::LC, LQ = K::LQ, LR = K::LR, KPL = K::KPL, KSTEP = K::KSTEP;
    constexpr int SZ = K::SZ, NK = K::NK, RT = K::RT, MT = K::MT, NW = K::NW, XC = K::XC;
    static_assert(QB <= 64 && QB % KSTEP == 0 && QB % 16 == 0, "block length");
    static_assert(N % KSTEP == 0 && N % 16 == 0 && P % 16 == 0 && P % XC == 0, "shape");

    __shared__ __attribute__((aligned(16))) TI smem[K::BUF_ELEMS];
    // per-wave copies of the block's per-token scalars (each wave computes its own)
    __shared__ __attribute__((aligned(16))) cum_t sCum[NW][64];   // cumulative log2 decay
    __shared__ __attribute__((aligned(16))) float sRow[NW][64];   // read-out row scale
    __shared__ __attribute__((aligned(16))) float sV[NW][64];     // exp2(cum at end of the token's 16-tile - cum)
    __shared__ __attribute__((aligned(16))) float sWx[NW][64];    // end-state weight exp2(cum_end - cum) (dt)
    __shared__ __attribute__((aligned(16))) float sDtf[NW][64];   // dt (Euler input scaling)
    __shared__ int sSeg[NW][64];
    __shared__ int sStart[NW][65];
    __shared__ int sSeqOf[NW][65];

    TI* sC = smem + K::OFF_C;
    TI* sBt = smem + K::OFF_BT;
    TI* sLm = smem + K::OFF_LM;
    TI* sXr = smem + K::OFF_XR;
    TI* sXw = smem + K::OFF_XW;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    // Work-item order: runs of consecutive (row, head) items go to the same
    // XCD (workgroups are dealt round-robin over the 8 XCDs), so the heads of
    // a row share that row's C, CB and B^T tiles in one L2.
    const int64_t units = prm.batch * prm.H;
    int64_t u = blockIdx.x;
    if (units % 8 == 0) u = (int64_t)(blockIdx.x % 8) * (units / 8) + blockIdx.x / 8;
    const int64_t b = u / prm.H, h = u % prm.H;
    const int64_t g = h / (prm.H / prm.G);
    const int64_t T = prm.T, H = prm.H, G = prm.G;
    const int nblk = prm.nblk;
    const int p0 = 16 * w;

    // A_h in log2 units, so that every decay is exp2 of a cumulative sum
    cum_t A2;
    if constexpr (sizeof(cum_t) == 8) A2 = -exp((double)prm.A_log[h]) * 1.4426950408889634;
    else A2 = -expf(prm.A_log[h]) * 1.4426950408889634f;
    const float Dh = prm.D ? prm.D[h] : 0.f;
    const int32_t* seqg = SEQ ? prm.seq_idx + b * T : nullptr;
    auto clamp_seq = [&](int s) { return s < 0 ? 0 : (s >= prm.nseqs ? (int)prm.nseqs - 1 : s); };

    // byte strides between consecutive tokens (the host keeps QB of them below 2^31)
    const int xs = (int)(H * P * SZ), ys = (int)(H * P * 4), cs = (int)(G * N * SZ), ds = (int)(H * 4);
    // row bases; block blk starts QB tokens further, and everything past the
    // row's last token reads as zero / is not written (buffer range check)
    const char* xrow = (const char*)prm.x + ((b * T) * H + h) * P * SZ;
    const char* yrow = (const char*)prm.y + ((b * T) * H + h) * P * 4;
    const char* crow = (const char*)prm.C + ((b * T) * G + g) * N * SZ;
    const char* drow = (const char*)prm.dt + ((b * T) * H + h) * 4;
    const char* btb0 = (const char*)prm.bt + ((b * G + g) * nblk) * (int64_t)N * QB * SZ;
    const char* cbb0 = (const char*)prm.cb + ((b * G + g) * nblk) * (int64_t)QB * QB * 4;
    const int64_t xrec = ((T - 1) * H + 1) * P * SZ, yrec = ((T - 1) * H + 1) * P * 4;
    const int64_t crec = ((T - 1) * G + 1) * N * SZ, drec = ((T - 1) * H + 1) * 4;

    // ---- initial state of the row's first sequence (S^T tiles, rows nrow(m, 4*lg+i))
    int prevseq = (int)b;
    if (SEQ && T > 0) prevseq = clamp_seq(seqg[0]);
    f32x4 st[MT];
    if (prm.init) {
        const float* src = prm.init + (((int64_t)prevseq * H + h) * P + p0 + lr) * N;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const float4 v = *(const float4*)(src + nrow<N>(m, 4 * lg));
            st[m] = f32x4{v.x, v.y, v.z, v.w};
        }
    } else {
#pragma unroll
        for (int m = 0; m < MT; ++m) st[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    auto write_state = [&](const f32x4 (&s)[MT], int seq) {
        if (!prm.fin) return;
        float* dst = prm.fin + (((int64_t)seq * H + h) * P + p0 + lr) * N;
#pragma unroll
        for (int m = 0; m < MT; ++m)
            *(float4*)(dst + nrow<N>(m, 4 * lg)) = make_float4(s[m][0], s[m][1], s[m][2], s[m][3]);
    };

    // The upper 16x16 tile next to an even diagonal tile is read by a 32-wide
    // K step of the diagonal product; it is zero and never rewritten.
    if constexpr (KSTEP > 16) {
        for (int v = tid; v < (RT / 2) * 16 * 16; v += NT) {
            const int r = 2 * (v / 256), i = (v / 16) % 16, c = v % 16;
            sLm[(16 * r + i) * LQ + 16 * (r + 1) + c] = to_in<TI>(0.f);
        }
    }

    // ---- one block of loads, issued at the top of an iteration and consumed
    // at its bottom (after the MFMA phase of the previous block), so no load
    // result lives across the loop back-edge and the wait counts stay exact.
    uint4 cr[K::CPT], br[K::BPT];
    float4 cbr[K::LMPT];
    uint2 xr[K::XPT][4];
    float dtv = 0.f;
    int sqv = 0;
    // Causal tile of each of this thread's L o CB pieces (row tile I, column tile
    // J <= I); the tile index v / 64 is uniform over the wave.
    int tI[K::LMPT], tJ[K::LMPT];
#pragma unroll
    for (int j = 0; j < K::LMPT; ++j) {
        const int q = (tid + j * NT) / 64;
        int I = 0;
        while ((I + 1) * (I + 2) / 2 <= q) ++I;
        tI[j] = I;
        tJ[j] = q - I * (I + 1) / 2;
    }
    auto issue = [&](int blk) {
        const int64_t t0 = (int64_t)blk * QB;
        const rsrc_t rx = make_rsrc(xrow + t0 * xs, xrec - t0 * xs);
        const rsrc_t rc = make_rsrc(crow + t0 * cs, crec - t0 * cs);
        const rsrc_t rd = make_rsrc(drow + t0 * ds, drec - t0 * ds);
        const rsrc_t rb = make_rsrc(btb0 + (int64_t)blk * N * QB * SZ, (int64_t)N * QB * SZ);
        const rsrc_t rcb = make_rsrc(cbb0 + (int64_t)blk * QB * QB * 4, (int64_t)QB * QB * 4);
        dtv = buf_load_f32(rd, lane * ds);
        if constexpr (SEQ) sqv = buf_load_i32(make_rsrc(seqg + t0, (T - t0) * 4), lane * 4);
#pragma unroll
        for (int j = 0; j < K::XPT; ++j) {
            const int v = tid + j * NT;
            const int q4 = v / (P / XC), c4 = v % (P / XC);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (K::XU % NT == 0 || v < K::XU) xr[j][e] = buf_load8(rx, (4 * q4 + e) * xs + c4 * 8);
        }
#pragma unroll
        for (int j = 0; j < K::CPT; ++j) {
            const int v = tid + j * NT;
            if (K::CV % NT == 0 || v < K::CV) cr[j] = buf_load16(rc, (v / (N / VE)) * cs + (v % (N / VE)) * 16);
        }
#pragma unroll
        for (int j = 0; j < K::BPT; ++j) {
            const int v = tid + j * NT;
            if (K::BV % NT == 0 || v < K::BV) br[j] = buf_load16(rb, v * 16);
        }
#pragma unroll
        for (int j = 0; j < K::LMPT; ++j) {
            const int v = tid + j * NT;
            if (K::LMU % NT == 0 || v < K::LMU) {
                const int t = 16 * tI[j] + (v % 64) / 4, s0 = 16 * tJ[j] + 4 * (v % 4);
                cbr[j] = __builtin_bit_cast(float4, buf_load16(rcb, (t * QB + s0) * 4));
            }
        }
    };

    // per-block values handed from the preparation of a block to its MFMA phase
    int nstart_c = 0, lastseq_c = prevseq;
    float cend_f = 0.f;

    // ---- preparation of a block from the issued loads: tiles into LDS, the
    //      within-block cumulative decay, segments, L o CB, X^T and weighted X^T
    auto prep = [&](int blk) {
        const int rows = (int)min((int64_t)QB, T - (int64_t)blk * QB);
#pragma unroll
        for (int j = 0; j < K::CPT; ++j) {
            const int v = tid + j * NT;
            if (K::CV % NT == 0 || v < K::CV) *(uint4*)(sC + (v / (N / VE)) * LC + (v % (N / VE)) * VE) = cr[j];
        }
#pragma unroll
        for (int j = 0; j < K::BPT; ++j) {
            const int v = tid + j * NT;
            if (K::BV % NT == 0 || v < K::BV) *(uint4*)(sBt + (v / (QB / VE)) * LQ + K::bt_col(v / (QB / VE), (v % (QB / VE)) * VE)) = br[j];
        }
        // per-token scalars, computed by every wave for itself (lane = token)
        const cum_t cum = wave_incl_scan((cum_t)dtv * A2);        // dt = 0 past the row's end
        const cum_t cend = __shfl(cum, QB - 1);
        const cum_t c16 = __shfl(cum, lane | 15);                // cum at the end of this token's 16-tile
        int nstart = 0;
        int segl = 0;
        cum_t before = 0;
        if constexpr (SEQ) {
            const int raw = clamp_seq(sqv);
            const int lastv = __shfl(raw, rows - 1);
            const int sq = lane < rows ? raw : lastv;            // padding tokens continue the last sequence
            const int up = __shfl_up(sq, 1);
            const int prev = (lane == 0) ? prevseq : up;
            const bool start = lane < rows && sq != prev;
            const uint64_t mask = __ballot(start);
            nstart = __popcll(mask);
            lastseq_c = __shfl(sq, QB - 1);
            if (nstart > 0) {
                const uint64_t upto = (lane == 63) ? ~0ull : ((2ull << lane) - 1ull);
                segl = __popcll(mask & upto);
                if (lane < QB) sSeg[w][lane] = segl;
                if (start) {
                    sStart[w][segl] = lane;
                    sSeqOf[w][segl] = sq;
                }
                if (lane == 0) {
                    sStart[w][0] = 0;
                    sSeqOf[w][0] = prevseq;
                }
            }
        }
        nstart_c = nstart;
        cend_f = (float)cend;
        const float dtf = EULER ? dtv : 1.f;
        if (lane < QB) {
            sCum[w][lane] = cum;
            sV[w][lane] = fast_exp2((float)(c16 - cum));
            sWx[w][lane] = fast_exp2((float)(cend - cum)) * dtf;
            if constexpr (EULER) sDtf[w][lane] = dtv;
        }
        wave_sync();
        if constexpr (SEQ) {
            if (nstart > 0) {
                const int a = sStart[w][segl];
                if (a > 0) before = sCum[w][a - 1];
            }
        }
        if (lane < QB) sRow[w][lane] = fast_exp2((float)(cum - before));

        // masked decay times C B^T over the causal tiles, 4 consecutive tokens s per piece:
        //   diagonal tile:  exp2(cum_t - cum_s) CB[t][s] for s <= t, else 0
        //   below it:       exp2(cum_t - cum_r) exp2(cum_r - cum_s) CB[t][s], r = last token of s's tile
        // (times dt_s with Euler input scaling; zero across sequence segments)
#pragma unroll
        for (int j = 0; j < K::LMPT; ++j) {
            const int v = tid + j * NT;
            if (K::LMU % NT == 0 || v < K::LMU) {
                const int I = tI[j], J = tJ[j];                 // uniform over the wave
                const int t = 16 * I + (v % 64) / 4, s0 = 16 * J + 4 * (v % 4);
                const float cb4[4] = {cbr[j].x, cbr[j].y, cbr[j].z, cbr[j].w};
                const cum_t ct = sCum[w][t];
                float val[4];
                if (I == J) {
                    cum_t c4[4];
                    if constexpr (sizeof(cum_t) == 4) {
                        const float4 cc = *(const float4*)(&sCum[w][s0]);
                        c4[0] = cc.x; c4[1] = cc.y; c4[2] = cc.z; c4[3] = cc.w;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) c4[e] = sCum[w][s0 + e];
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float lv = fast_exp2((float)(ct - c4[e])) * cb4[e];
                        val[e] = (s0 + e <= t) ? lv : 0.f;
                    }
                } else {
                    const float ut = fast_exp2((float)(ct - sCum[w][16 * J + 15]));
                    const float4 v4 = *(const float4*)(&sV[w][s0]);
                    val[0] = ut * v4.x * cb4[0];
                    val[1] = ut * v4.y * cb4[1];
                    val[2] = ut * v4.z * cb4[2];
                    val[3] = ut * v4.w * cb4[3];
                }
                if constexpr (EULER) {
                    const float4 d4 = *(const float4*)(&sDtf[w][s0]);
                    val[0] *= d4.x; val[1] *= d4.y; val[2] *= d4.z; val[3] *= d4.w;
                }
                if constexpr (SEQ) {
                    if (nstart > 0) {
                        const int segt = sSeg[w][t];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (sSeg[w][s0 + e] != segt) val[e] = 0.f;
                    }
                }
                if constexpr (sizeof(TI) == 2) {
                    *(bf16x4*)(sLm + t * LQ + s0) = bf16x4{(__bf16)val[0], (__bf16)val[1], (__bf16)val[2], (__bf16)val[3]};
                } else {
                    *(float4*)(sLm + t * LQ + s0) = make_float4(val[0], val[1], val[2], val[3]);
                }
            }
        }
        // X (row-major) and, for single-segment blocks, the end-state weighted X
#pragma unroll
        for (int j = 0; j < K::XPT; ++j) {
            const int v = tid + j * NT;
            if (K::XU % NT == 0 || v < K::XU) {
                const int q4 = v / (P / XC), c4 = v % (P / XC);
                const int t0l = 4 * q4;
                const float4 w4 = *(const float4*)(&sWx[w][t0l]);
                const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    *(uint2*)(sXr + (t0l + e) * LR + c4 * XC) = xr[j][e];
                    if (!SEQ || nstart == 0) {
                        TI wx[XC];
#pragma unroll
                        for (int k = 0; k < XC; ++k) wx[k] = to_in<TI>(wv[e] * to_f32(((const TI*)&xr[j][e])[k]));
                        uint2 pk;
                        __builtin_memcpy(&pk, wx, 8);
                        *(uint2*)(sXw + (t0l + e) * LR + c4 * XC) = pk;
                    }
                }
            }
        }
    };

    auto mfma_phase = [&](int blk) {
        const int nstart = nstart_c;
        // ---- MFMA phase, outputs transposed: y^T tiles (rows p0..p0+15, columns t)
        frag sf[NK];
        state_frags<N>(st, sf);
        f32x4 acc_y[RT], acc_o[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            acc_y[r] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc_o[r] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        constexpr int KS = QB / KSTEP;           // K steps over the tokens of a block
        // B^T fragment (state tile m, K step ks): row nrow(m, lr) = nrow(m, 0) + nrow(0, lr),
        // and the row swizzle depends on the lane only (bit 3 of nrow(0, lr)), so every
        // fragment is a per-K-step lane base plus a compile-time row offset
        const TI* bt_lane[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            bt_lane[ks] = sBt + nrow<N>(0, lr) * LQ + K::bt_col(nrow<N>(0, lr), ks * KSTEP + KPL * lg);
        auto bt_frag = [&](int m, int ks) { return lds_frag<TI>(bt_lane[ks / KSTEP] + nrow<N>(m, 0) * LQ); };
        // diagonal block: (L o CB) X, as X^T (L o CB)^T; token tile r only needs s < 16 (r + 1)
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int ks = 0; ks < 16 * (r + 1); ks += KSTEP)
                acc_y[r] = MF::mma(x_frag(sXr, LR, ks, p0, lr, lg),
                                   lds_frag<TI>(sLm + (16 * r + lr) * LQ + ks + KPL * lg), acc_y[r]);
        if (!SEQ || nstart == 0) {
            // carried state read out by C:  S C^T
#pragma unroll
            for (int r = 0; r < RT; ++r)
#pragma unroll
                for (int k = 0; k < NK; ++k)
                    acc_o[r] = MF::mma(sf[k], c_frag<N>(sC + (16 * r + lr) * LC, k, lg), acc_o[r]);
            // state <- exp(cum_end) state + B^T (weighted X)
            const float alpha = fast_exp2(cend_f);
#pragma unroll
            for (int m = 0; m < MT; ++m) st[m] *= alpha;
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) st[m] = MF::mma(bt_frag(m, ks * KSTEP), x_frag(sXw, LR, ks * KSTEP, p0, lr, lg), st[m]);
#pragma unroll
            for (int r = 0; r < RT; ++r) acc_o[r] *= sRow[w][16 * r + lr];
        } else if constexpr (SEQ) {
            // ---- block with sequence starts, one segment at a time
            // (1) read-out of each segment's incoming state
            for (int j = 0; j <= nstart; ++j) {
                const int a = sStart[w][j];
                const int e = (j < nstart) ? sStart[w][j + 1] - 1 : QB - 1;
                if (e < a) continue;                         // empty first segment
                frag f[NK];
                if (j == 0) {
#pragma unroll
                    for (int k = 0; k < NK; ++k) f[k] = sf[k];
                } else if (prm.init) {
                    global_state_frags<N>(prm.init + (((int64_t)sSeqOf[w][j] * H + h) * P + p0 + lr) * N, lg, f);
                } else {
                    continue;                                // a zero initial state reads out nothing
                }
#pragma unroll
                for (int r = 0; r < RT; ++r) {
                    f32x4 tmp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int k = 0; k < NK; ++k) tmp = MF::mma(f[k], c_frag<N>(sC + (16 * r + lr) * LC, k, lg), tmp);
                    const int t = 16 * r + lr;
                    const float sc = (sSeg[w][t] == j) ? sRow[w][t] : 0.f;
                    acc_o[r] += sc * tmp;
                }
            }
            // (2) state at the end of each segment: a sequence that ends inside
            //     the block hands its state to final_state; the last segment's
            //     state is carried on
            if (sStart[w][1] == 0) write_state(st, sSeqOf[w][0]);   // previous sequence ended with the previous block
            for (int j = 0; j <= nstart; ++j) {
                const int a = sStart[w][j];
                const int e = (j < nstart) ? sStart[w][j + 1] - 1 : QB - 1;
                if (e < a) continue;
                block_sync_lds();                             // the previous segment's weighted X is consumed
                for (int v = tid; v < P * QB; v += NT) {
                    const int t = v / P, pr = v % P;
                    const float ws = (sSeg[w][t] == j)
                        ? fast_exp2((float)(sCum[w][e] - sCum[w][t])) * (EULER ? sDtf[w][t] : 1.f) : 0.f;
                    sXw[t * LR + pr] = to_in<TI>(ws * to_f32(sXr[t * LR + pr]));
                }
                block_sync_lds();
                const cum_t before = (a == 0) ? (cum_t)0 : sCum[w][a - 1];
                const float carry = fast_exp2((float)(sCum[w][e] - before));
                f32x4 F[MT];
                if (j == 0) {
#pragma unroll
                    for (int m = 0; m < MT; ++m) F[m] = st[m] * carry;
                } else if (prm.init) {
                    const float* src = prm.init + (((int64_t)sSeqOf[w][j] * H + h) * P + p0 + lr) * N;
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        const float4 iv = *(const float4*)(src + nrow<N>(m, 4 * lg));
                        F[m] = f32x4{iv.x, iv.y, iv.z, iv.w} * carry;
                    }
                } else {
#pragma unroll
                    for (int m = 0; m < MT; ++m) F[m] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int ks = 0; ks < QB; ks += KSTEP)
                        F[m] = MF::mma(lds_frag<TI>(sBt + nrow<N>(m, lr) * LQ + K::bt_col(nrow<N>(m, lr), ks + KPL * lg)),
                                       x_frag(sXw, LR, ks, p0, lr, lg), F[m]);
                if (j < nstart) {
                    write_state(F, sSeqOf[w][j]);
                } else {
#pragma unroll
                    for (int m = 0; m < MT; ++m) st[m] = F[m];
                }
            }
            // Settle this rare path's own memory traffic here, so that the
            // common path's wait counts stay exact (prefetches stay in flight).
            __builtin_amdgcn_s_waitcnt(0);
        }

        // ---- y = read-out + diagonal block + D x: lane holds y[t = 16r + lr][p0 + 4lg .. +3],
        //      one 16-byte store per token tile (past-the-end tokens are dropped by the range check)
        const int64_t t0 = (int64_t)blk * QB;
        const rsrc_t ry = make_rsrc(yrow + t0 * ys, yrec - t0 * ys);
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const int t = 16 * r + lr;
            f32x4 out = acc_o[r] + acc_y[r];
            {
                float xv[4];
                if constexpr (sizeof(TI) == 2) {
                    const bf16x4 x4 = *(const bf16x4*)(sXr + t * LR + p0 + 4 * lg);
#pragma unroll
                    for (int i = 0; i < 4; ++i) xv[i] = (float)x4[i];
                } else {
                    const float4 x4 = *(const float4*)(sXr + t * LR + p0 + 4 * lg);
                    xv[0] = x4.x; xv[1] = x4.y; xv[2] = x4.z; xv[3] = x4.w;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) out[i] += Dh * xv[i];
            }
            buf_store16(out, ry, t * ys + (p0 + 4 * lg) * 4);
        }
        if constexpr (SEQ) prevseq = lastseq_c;
    };

    if (nblk > 0) {
        issue(0);
        prep(0);
        block_sync_lds();
    }
    // The initial state (loaded at entry) is carried through the loop; settle
    // its loads here so the loop header does not wait on memory each iteration.
    __builtin_amdgcn_s_waitcnt(0);
    for (int blk = 0; blk < nblk; ++blk) {
        if (blk + 1 < nblk) issue(blk + 1);
        mfma_phase(blk);
        if (blk + 1 < nblk) {
            block_sync_lds();        // block blk's tiles are no longer read
            prep(blk + 1);
            block_sync_lds();        // block blk+1's tiles are complete
        }
    }
    // the state after the row's last token belongs to its last sequence
    if (T > 0 || !SEQ) write_state(st, prevseq);
}

}  // namespace ssd
