// Host side of ssd_backward (declared in include/ssd.h): argument checks, the
// workspace layout and the launches of the backward kernels.  Every check runs
// before the first HIP call.
#include "ssd.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "ssd_bwd.hpp"
#include "ssd_host.hpp"
#include "ssd_launch.hpp"

namespace ssd {
// dB or dC of a group = the sum of its heads' contributions (fp32 or bf16), in
// head order, in fp32.  One thread per 8 consecutive outputs; the loads of four
// heads are issued before their sums, so each thread keeps several in flight.
struct F8 {
    float v[8];
};
__device__ inline F8 load8(const float* p) {
    const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
    return F8{{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w}};
}
__device__ inline F8 load8(const __bf16* p) {
    const uint4 u = *(const uint4*)p;
    F8 r;
    const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        r.v[2 * k] = __uint_as_float(w[k] << 16);
        r.v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
    return r;
}
template <typename S>
__global__ __launch_bounds__(256) void ssd_bwd_group_sum_kernel(const S* __restrict__ src, float* __restrict__ dst,
                                                                int64_t rows, int H, int G, int N) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;        // 8-wide chunk of dst
    const int n8 = N / 8;
    const int64_t total = rows * G * n8;
    if (i >= total) return;
    const int64_t bt = i / (G * n8);
    const int g = (int)((i / n8) % G), c = (int)(i % n8);
    const int hpg = H / G;
    const S* s = src + (bt * H + (int64_t)g * hpg) * N + 8 * c;
    float acc[8];
    const F8 first = load8(s);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = first.v[k];
    int j = 1;
    for (; j + 4 <= hpg; j += 4) {
        F8 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = load8(s + (int64_t)(j + u) * N);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] += v[u].v[k];
    }
    for (; j < hpg; ++j) {
        const F8 v = load8(s + (int64_t)j * N);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] += v.v[k];
    }
    float4* d = (float4*)(dst + 8 * i);
    d[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    d[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// dt (b, T, H) -> (b, H, T): the backward kernels read each (row, head)'s step
// sizes as one contiguous run per block.  32 x 32 tiles through LDS, so that
// both the reads (along heads) and the writes (along tokens) are contiguous;
// workgroup (x, y) = (row and token tile, head tile).
__global__ __launch_bounds__(256) void ssd_transpose_dt_kernel(const float* __restrict__ dt, float* __restrict__ dtT,
                                                               int64_t batch, int64_t T, int64_t H) {
    __shared__ float tile[32][33];
    const int64_t ntt = (T + 31) / 32;
    const int64_t b = (int64_t)blockIdx.x / ntt, t0 = ((int64_t)blockIdx.x % ntt) * 32, h0 = (int64_t)blockIdx.y * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    if (b >= batch) return;                                       // (uniform over the workgroup)
    for (int k = ty; k < 32; k += 8) {
        const int64_t t = t0 + k, h = h0 + tx;
        tile[k][tx] = (t < T && h < H) ? dt[(b * T + t) * H + h] : 0.f;
    }
    __syncthreads();
    for (int k = ty; k < 32; k += 8) {
        const int64_t h = h0 + k, t = t0 + tx;
        if (h < H && t < T) dtT[(b * H + h) * T + t] = tile[tx][k];
    }
}

// Per-head scalars: sums over rows or packed sequences (in order) of the reverse pass's partial sums.
__global__ __launch_bounds__(256) void ssd_bwd_scalars_kernel(const float* __restrict__ part,
                                                              const float* __restrict__ A_log, int64_t batch, int H,
                                                              float* dA_log, float* ddt_bias, float* dD) {
    const int h = blockIdx.x * 256 + threadIdx.x;
    if (h >= H) return;
    float a = 0.f, bb = 0.f, d = 0.f;
    for (int64_t r = 0; r < batch; ++r) {
        const float* q = part + (r * H + h) * 3;
        a += q[0];
        bb += q[1];
        d += q[2];
    }
    dA_log[h] = a * -expf(A_log[h]);      // dA/dA_log = A
    if (ddt_bias) ddt_bias[h] = bb;
    if (dD) dD[h] = d;
}

// The table of packed sequences: each token that starts or ends its sequence
// writes the sequence's row and first or end token (ids clamped to 0..nseqs-1;
// ids that are not nondecreasing or repeat across rows give meaningless but
// in-range entries).  Entries are (row, first token, end token, first hin slot).
__global__ __launch_bounds__(256) void ssd_seq_table_kernel(const int32_t* __restrict__ seq, int64_t batch, int64_t T,
                                                            int64_t nseqs, int64_t* __restrict__ tab) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= batch * T) return;
    const int64_t r = i / T, t = i % T;
    auto id = [&](int64_t u) {
        const int64_t v = seq[r * T + u];
        return v < 0 ? (int64_t)0 : (v >= nseqs ? nseqs - 1 : v);
    };
    const int64_t k = id(t);
    if (t == 0 || id(t - 1) != k) {
        tab[4 * k + 0] = r;
        tab[4 * k + 1] = t;
    }
    if (t == T - 1 || id(t + 1) != k) tab[4 * k + 2] = t + 1;
}
// First hin slot of each sequence: the running count of blocks of the sequences
// before it (a sequence that would not fit the slots is given no tokens).
__global__ __launch_bounds__(64) void ssd_seq_slots_kernel(int64_t* tab, int64_t nseqs, int64_t qb, int64_t cap) {
    if (threadIdx.x != 0) return;
    int64_t off = 0;
    for (int64_t k = 0; k < nseqs; ++k) {
        int64_t* e = tab + 4 * k;
        const int64_t len = e[2] > e[1] ? e[2] - e[1] : 0;
        const int64_t nb = (len + qb - 1) / qb;
        if (off + nb > cap) {
            e[2] = e[1];
            e[3] = 0;
            continue;
        }
        e[3] = off;
        off += nb;
    }
}

// Gradient with respect to the end state of every row segment but the last,
// written over the reverse local pass's results: G(S-1) = dfinal and
// G(j) = carry(j+1) G(j+1) + local(j+1), where slot j holds segment j+1's local
// gradient and decay.  One thread per 4 consecutive state elements.
__global__ __launch_bounds__(256) void ssd_bwd_kcombine_kernel(const float* __restrict__ dfinal, float* seg_grad,
                                                               const float* __restrict__ kcarry, int64_t rows_heads,
                                                               int64_t pn, int nseg) {
    const int64_t pn4 = pn / 4;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t bh = idx / pn4, e = idx % pn4;
    if (bh >= rows_heads) return;
    const int s1 = nseg - 1;
    float4 st = dfinal ? *(const float4*)(dfinal + bh * pn + 4 * e) : make_float4(0.f, 0.f, 0.f, 0.f);
    float4* base = (float4*)(seg_grad + bh * s1 * pn) + e;
    const float* carry = kcarry + bh * s1;
    // eight segments' loads in flight before their (sequential) combine
    for (int j0 = s1 - 1; j0 >= 0; j0 -= 8) {
        float4 l[8];
        float c[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (j0 - k >= 0) {
                l[k] = base[(j0 - k) * (pn / 4)];
                c[k] = carry[j0 - k];
            }
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (j0 - k >= 0) {
                st = make_float4(c[k] * st.x + l[k].x, c[k] * st.y + l[k].y, c[k] * st.z + l[k].z, c[k] * st.w + l[k].w);
                base[(j0 - k) * (pn / 4)] = st;
            }
        }
    }
}

// Fill / copy for the degenerate cases (no token): dinit = dfinal or 0, scalars 0.
__global__ __launch_bounds__(256) void ssd_fill_kernel(float* dst, const float* src, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

}  // namespace ssd

namespace {

using namespace ssd_host;

// Tokens per block of the backward kernels.
int bwd_block(const ssd_problem_t* p) { return p->dtype == SSD_DTYPE_BF16 ? ssd::bwd_block_bf16() : ssd::bwd_block_f32(); }

// Segments per row (rows without sequence ids).  With at most 128 (row, head)
// items, rows are cut into up to 512 / items segments of whole 64-token blocks,
// down to 4 blocks per segment, as the forward does.  With more items, the count
// S <= 8 that minimises the rounds of workgroups over the 256 CUs per unit of
// row length, ceil(items S / 256) / S, plus a charge of 0.5 (S - 1) / S for the
// local passes (measured on MI355X: 320 items run best as 4 segments, 192 unsplit).
// The problem's `segments` field, when positive, forces the count (as for the
// forward; without sequence ids).  A function of the problem alone, so the
// workspace size is known on the host.
struct BwdSegs {
    int nseg;
    int64_t seg_tokens;
};
BwdSegs bwd_segments(const ssd_problem_t* p) {
    const int64_t nb64 = (p->seqlen + 63) / 64;
    BwdSegs r{1, std::max<int64_t>(p->seqlen, 1)};
    if (nb64 <= 1 || p->batch == 0) return r;
    int64_t S = 1;
    if (p->segments > 0) {
        S = p->segments;
    } else {
        const int64_t units = p->batch * p->nheads;
        if (units <= 128) {
            S = std::min<int64_t>(512 / units, nb64 / 4);
        } else {
            double best = 1e30;
            for (int64_t c = 1; c <= 8 && (c == 1 || nb64 / c >= 4); ++c) {
                const double cost = double((units * c + 255) / 256) / double(c) + 0.5 * double(c - 1) / double(c);
                if (cost < best - 1e-9) {
                    best = cost;
                    S = c;
                }
            }
        }
    }
    S = std::max<int64_t>(1, std::min<int64_t>(S, nb64));
    if (S == 1) return r;
    r.seg_tokens = (nb64 + S - 1) / S * 64;
    r.nseg = (int)((p->seqlen + r.seg_tokens - 1) / r.seg_tokens);
    if (r.nseg == 1) r.seg_tokens = p->seqlen;
    return r;
}

// Workspace of the backward pass: a per-token scalar and dt, both (b, H, T); each
// block's incoming state in the input type, (H, slots, P, N) with
// slots = b * blocks per row + nseqs (enough for any split of the rows into
// sequences, each sequence starting a new block); the per-sequence scalar sums
// (nseqs, H, 3); the table of packed sequences (nseqs x 4 int64); and, when a
// group has more than one head, each head's dB and dC contribution (b, T, H, N)
// in the input type before the sum over the group.
struct BwdWs {
    int64_t q_off, dt_off, hin_off, part_off, tab_off, seg_off, segc_off, grad_off, gradc_off, dbh_off, dch_off, total,
        hin_slots;
};
BwdWs bwd_ws_layout(const ssd_problem_t* p) {
    BwdWs l;
    const BwdSegs sg = bwd_segments(p);
    const int64_t bth = p->batch * p->seqlen * p->nheads;
    const int64_t items = std::max(std::max(p->nseqs, p->batch), p->batch * sg.nseg);
    const bool per_head = p->ngroups != p->nheads;
    const int qb = bwd_block(p);
    const int64_t nblk = (p->seqlen + qb - 1) / qb;
    l.hin_slots = std::max(p->batch * nblk + p->nseqs, p->batch * sg.nseg * ((sg.seg_tokens + qb - 1) / qb));
    l.q_off = 0;
    l.dt_off = align256(bth * 4);
    l.hin_off = l.dt_off + align256(bth * 4);
    l.part_off = l.hin_off + align256(p->nheads * l.hin_slots * p->headdim * p->dstate * elem_size(p->dtype));
    l.tab_off = l.part_off + align256(items * p->nheads * 12);
    // split rows: incoming states and their decays (forward local pass), then the
    // gradients at segment ends and their decays (reverse local pass)
    const int64_t nsl = p->batch * p->nheads * (sg.nseg - 1);
    l.seg_off = l.tab_off + align256(p->nseqs * 32);
    l.segc_off = l.seg_off + align256(nsl * p->headdim * p->dstate * 4);
    l.grad_off = l.segc_off + align256(nsl * 4);
    l.gradc_off = l.grad_off + align256(nsl * p->headdim * p->dstate * 4);
    l.dbh_off = l.gradc_off + align256(nsl * 4);
    const int64_t hn = per_head ? align256(bth * p->dstate * elem_size(p->dtype)) : 0;
    l.dch_off = l.dbh_off + hn;
    l.total = l.dch_off + hn;
    return l;
}

}  // namespace

extern "C" {

size_t ssd_backward_workspace_size(const ssd_problem_t* p) {
    if (ssd_validate(p) != SSD_OK) return 0;
    return (size_t)bwd_ws_layout(p).total;
}

int ssd_backward(const ssd_problem_t* p, const void* x, const float* dt, const float* dt_bias, const float* A_log,
                 const void* B, const void* C, const float* D, const float* init_state, const int32_t* seq_idx,
                 const float* dy, const float* dfinal, float* dx, float* ddt, float* dA_log, float* dB, float* dC,
                 float* dD, float* dinit, float* ddt_bias, void* workspace, size_t workspace_bytes, void* stream) {
    const int v = ssd_validate(p);
    if (v != SSD_OK) return v;
    if (!seq_idx && p->nseqs != p->batch) return SSD_ERR_BAD_SHAPE;
    if (seq_idx && p->batch > 0 && p->seqlen > 0 && p->nseqs < 1) return SSD_ERR_BAD_SHAPE;
    const int P = (int)p->headdim, N = (int)p->dstate;
    const bool bf = p->dtype == SSD_DTYPE_BF16;
    if (!(bf ? ssd::supported_bwd_bf16(P, N) : ssd::supported_bwd_f32(P, N))) return SSD_ERR_UNSUPPORTED;
    const bool tokens = p->batch > 0 && p->seqlen > 0;
    if (!A_log || !dA_log) return SSD_ERR_NULL_POINTER;
    if (tokens && (!x || !dt || !B || !C || !dy || !dx || !ddt || !dB || !dC)) return SSD_ERR_NULL_POINTER;
    const BwdWs wl = bwd_ws_layout(p);
    if (wl.total > 0 && tokens && !workspace) return SSD_ERR_WORKSPACE;
    if (tokens && static_cast<int64_t>(workspace_bytes) < wl.total) return SSD_ERR_WORKSPACE;
    if (misaligned(x, 16) || misaligned(B, 16) || misaligned(C, 16) || misaligned(dy, 16) || misaligned(dB, 16) ||
        misaligned(dC, 16) || misaligned(init_state, 16) || misaligned(dfinal, 16) || misaligned(dinit, 16) ||
        misaligned(dx, 16) || misaligned(dt, 4) || misaligned(ddt, 4) || misaligned(A_log, 4) ||
        misaligned(dA_log, 4) || misaligned(dt_bias, 4) || misaligned(ddt_bias, 4) || misaligned(D, 4) ||
        misaligned(dD, 4) || misaligned(seq_idx, 4) || misaligned(workspace, 256))
        return SSD_ERR_ALIGNMENT;
    // one block of tokens is addressed with 32-bit byte offsets
    const int qb = bwd_block(p);
    if (double(qb) * double(p->nheads) * double(std::max(p->headdim, p->dstate)) * 4.0 >= 2147483647.0)
        return SSD_ERR_BAD_SHAPE;
    const Sizes s = sizes(p);
    const int64_t hb = p->nheads * 4;
    const int64_t gbc = p->batch * p->seqlen * p->ngroups * p->dstate * 4;
    const void* in_ptr[] = {x, dt, dt_bias, A_log, B, C, D, init_state, dy, dfinal, workspace, seq_idx};
    const int64_t in_sz[] = {s.x, s.dt, hb, hb, s.bc, s.bc, hb, s.state, s.y, s.state, wl.total, s.seq};
    const void* out_ptr[] = {dx, ddt, dA_log, dB, dC, dD, dinit, ddt_bias};
    const int64_t out_sz[] = {s.y, s.dt, hb, gbc, gbc, hb, s.state, hb};
    for (int o = 0; o < 8; ++o) {
        for (int i = 0; i < 12; ++i)
            if (overlap(out_ptr[o], out_sz[o], in_ptr[i], in_sz[i])) return SSD_ERR_ALIAS;
        for (int o2 = o + 1; o2 < 8; ++o2)
            if (overlap(out_ptr[o], out_sz[o], out_ptr[o2], out_sz[o2])) return SSD_ERR_ALIAS;
    }
    const int d = check_device();
    if (d != SSD_OK) return d;
    hipStream_t st = static_cast<hipStream_t>(stream);
    auto fill = [&](float* dst, const float* src, int64_t n) {
        if (!dst || n <= 0) return hipSuccess;
        hipLaunchKernelGGL(ssd::ssd_fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, dst, src, n);
        return hipGetLastError();
    };
    hipError_t e = hipSuccess;
    if (!tokens) {
        // no token: final = init, so dinit = dfinal; every per-head sum is empty
        e = fill(dA_log, nullptr, p->nheads);
        if (e == hipSuccess) e = fill(dD, nullptr, p->nheads);
        if (e == hipSuccess) e = fill(ddt_bias, nullptr, p->nheads);
        // (a packed sequence that does not occur has no influence: dinit = 0)
        if (e == hipSuccess) e = fill(dinit, seq_idx ? nullptr : dfinal, p->nseqs * p->nheads * p->headdim * p->dstate);
        return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
    }
    char* ws = static_cast<char*>(workspace);
    const bool per_head = p->ngroups != p->nheads;
    ssd::BwdParams prm;
    prm.x = x;
    prm.dt = reinterpret_cast<float*>(ws + wl.dt_off);
    prm.dt_bias = dt_bias;
    prm.A_log = A_log;
    prm.B = B;
    prm.C = C;
    prm.D = D;
    prm.init = init_state;
    prm.dy = dy;
    prm.dfinal = dfinal;
    prm.dx = dx;
    prm.ddt = ddt;
    prm.dBh = per_head ? static_cast<void*>(ws + wl.dbh_off) : static_cast<void*>(dB);
    prm.dCh = per_head ? static_cast<void*>(ws + wl.dch_off) : static_cast<void*>(dC);
    prm.h_bf16 = per_head && bf ? 1 : 0;
    prm.dinit = dinit;
    prm.q = reinterpret_cast<float*>(ws + wl.q_off);
    prm.hin = ws + wl.hin_off;
    prm.part = reinterpret_cast<float*>(ws + wl.part_off);
    prm.batch = p->batch;
    prm.T = p->seqlen;
    prm.H = p->nheads;
    prm.G = p->ngroups;
    prm.HB = per_head ? p->nheads : p->ngroups;
    prm.nblk = (int)((p->seqlen + qb - 1) / qb);
    prm.hin_blocks = wl.hin_slots;
    prm.seqtab = seq_idx ? reinterpret_cast<const int64_t*>(ws + wl.tab_off) : nullptr;
    prm.dt_softplus = (p->flags & SSD_FLAG_DT_SOFTPLUS) ? 1 : 0;
    prm.x_scale = x_scale_of(p);
    const BwdSegs sg = seq_idx ? BwdSegs{1, p->seqlen} : bwd_segments(p);
    prm.nseg = sg.nseg;
    prm.seg_tokens = sg.seg_tokens;
    prm.seg_state = reinterpret_cast<const float*>(ws + wl.seg_off);
    prm.seg_grad = reinterpret_cast<const float*>(ws + wl.grad_off);
    const int64_t items = seq_idx ? p->nseqs : p->batch * sg.nseg;     // sequences, row segments or rows
    const int64_t grid = items * p->nheads;
    if (seq_idx) {
        int64_t* tab = reinterpret_cast<int64_t*>(ws + wl.tab_off);
        e = fill(reinterpret_cast<float*>(tab), nullptr, p->nseqs * 8);
        const int64_t n = p->batch * p->seqlen;
        if (e == hipSuccess) {
            hipLaunchKernelGGL(ssd::ssd_seq_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, seq_idx,
                               p->batch, p->seqlen, p->nseqs, tab);
            hipLaunchKernelGGL(ssd::ssd_seq_slots_kernel, dim3(1), dim3(64), 0, st, tab, p->nseqs, (int64_t)qb,
                               wl.hin_slots);
            e = hipGetLastError();
        }
    }
    if (e == hipSuccess) {
        const dim3 grid((unsigned)(p->batch * ((p->seqlen + 31) / 32)), (unsigned)((p->nheads + 31) / 32));
        hipLaunchKernelGGL(ssd::ssd_transpose_dt_kernel, grid, dim3(256), 0, st, dt,
                           const_cast<float*>(prm.dt), p->batch, p->seqlen, p->nheads);
        e = hipGetLastError();
    }
    if (e == hipSuccess && sg.nseg > 1) {
        // forward state entering each segment: the forward's local pass and combine step
        ssd::ScanParams sp;
        sp.x = x;
        sp.dt = dt;
        sp.A_log = A_log;
        sp.D = D;
        sp.init = init_state;
        sp.seq_idx = nullptr;
        sp.y = nullptr;
        sp.fin = nullptr;
        sp.B = B;
        sp.C = C;
        sp.batch = p->batch;
        sp.T = p->seqlen;
        sp.H = p->nheads;
        sp.G = p->ngroups;
        sp.nseqs = p->batch;
        sp.nblk = (int)((p->seqlen + 63) / 64);
        sp.dt_bias = dt_bias;
        sp.dt_softplus = prm.dt_softplus;
        sp.x_scale = prm.x_scale;
        sp.seg_blocks = (int)(sg.seg_tokens / 64);
        sp.nseg = sg.nseg;
        sp.seg_state = reinterpret_cast<float*>(ws + wl.seg_off);
        sp.seg_carry = reinterpret_cast<float*>(ws + wl.segc_off);
        const int64_t lgrid = p->batch * p->nheads * (sg.nseg - 1);
        e = bf ? ssd::launch_scan_bf16(P, N, 64, false, prm.x_scale != 0, true, P / 16, sp, lgrid, st)
               : ssd::launch_scan_f32(P, N, 64, false, prm.x_scale != 0, true, P / 16, sp, lgrid, st);
        if (e == hipSuccess) {
            ssd::CombineParams cp;
            cp.init = init_state;
            cp.seq_idx = nullptr;
            cp.seg_state = sp.seg_state;
            cp.seg_carry = sp.seg_carry;
            cp.batch = p->batch;
            cp.T = p->seqlen;
            cp.H = p->nheads;
            cp.nseqs = p->batch;
            cp.P = P;
            cp.N = N;
            cp.nseg = sg.nseg;
            e = ssd::launch_combine(cp, st);
        }
        // gradient leaving each segment's end: the reverse local pass and combine step
        float* kloc = reinterpret_cast<float*>(ws + wl.grad_off);
        float* kcar = reinterpret_cast<float*>(ws + wl.gradc_off);
        if (e == hipSuccess)
            e = bf ? ssd::launch_bwd_klocal_bf16(P, N, prm, kloc, kcar, lgrid, st)
                   : ssd::launch_bwd_klocal_f32(P, N, prm, kloc, kcar, lgrid, st);
        if (e == hipSuccess) {
            const int64_t rh = p->batch * p->nheads, pn = (int64_t)P * N;
            const int64_t n = rh * pn / 4;
            hipLaunchKernelGGL(ssd::ssd_bwd_kcombine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                               dfinal, kloc, kcar, rh, pn, sg.nseg);
            e = hipGetLastError();
        }
    }
    if (e == hipSuccess)
        e = bf ? ssd::launch_bwd_bf16(P, N, prm, grid, st) : ssd::launch_bwd_f32(P, N, prm, grid, st);
    if (e == hipSuccess && per_head) {
        const int64_t rows = p->batch * p->seqlen;
        const int64_t n8 = rows * p->ngroups * N / 8;
        const unsigned blocks = (unsigned)((n8 + 255) / 256);
        if (prm.h_bf16) {
            hipLaunchKernelGGL(ssd::ssd_bwd_group_sum_kernel<__bf16>, dim3(blocks), dim3(256), 0, st,
                               (const __bf16*)prm.dBh, dB, rows, (int)p->nheads, (int)p->ngroups, N);
            hipLaunchKernelGGL(ssd::ssd_bwd_group_sum_kernel<__bf16>, dim3(blocks), dim3(256), 0, st,
                               (const __bf16*)prm.dCh, dC, rows, (int)p->nheads, (int)p->ngroups, N);
        } else {
            hipLaunchKernelGGL(ssd::ssd_bwd_group_sum_kernel<float>, dim3(blocks), dim3(256), 0, st,
                               (const float*)prm.dBh, dB, rows, (int)p->nheads, (int)p->ngroups, N);
            hipLaunchKernelGGL(ssd::ssd_bwd_group_sum_kernel<float>, dim3(blocks), dim3(256), 0, st,
                               (const float*)prm.dCh, dC, rows, (int)p->nheads, (int)p->ngroups, N);
        }
        e = hipGetLastError();
    }
    if (e == hipSuccess) {
        hipLaunchKernelGGL(ssd::ssd_bwd_scalars_kernel, dim3((unsigned)((p->nheads + 255) / 256)), dim3(256), 0, st,
                           prm.part, A_log, items, (int)p->nheads, dA_log, ddt_bias, dD);
        e = hipGetLastError();
    }
    if (log_enabled())
        std::fprintf(stderr, "[ssd] backward dtype=%d P=%d N=%d QB=%d grid=%lld segments=%d x %lld tokens per-head sums=%d -> %s\n",
                     p->dtype, P, N, qb, (long long)grid, sg.nseg, (long long)sg.seg_tokens, (int)per_head,
                     hipGetErrorString(e));
    return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

}  // extern "C"
