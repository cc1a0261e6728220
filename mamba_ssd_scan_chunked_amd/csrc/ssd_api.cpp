// Host side of the C ABI declared in include/ssd.h: argument checks, kernel
// selection and the launch.  Every check runs before the first HIP
// call, so invalid arguments are reported without touching the device.
#include "ssd.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstdio>

#include "ssd_host.hpp"
#include "ssd_kernels.hpp"
#include "ssd_launch.hpp"

#include <algorithm>
#include <mutex>

namespace ssd {
// Incoming state of every segment from the local pass: for each (row, head) and
// state element, S_in(0) = the row's initial state and
// S_in(s+1) = carry(s) S_in(s) + local(s), written over local(s) (the
// inter-chunk state recurrence real_end = block_decay * prev + local_end at
// segment granularity).  One thread per 4 consecutive elements.
__global__ __launch_bounds__(256) void ssd_combine_kernel(CombineParams prm) {
    const int64_t pn4 = (int64_t)prm.P * prm.N / 4;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t bh = idx / pn4, e = idx % pn4;
    if (bh >= prm.batch * prm.H) return;
    const int64_t b = bh / prm.H, h = bh % prm.H;
    float4 st = make_float4(0.f, 0.f, 0.f, 0.f);
    if (prm.init) {
        int64_t seq0 = b;
        if (prm.seq_idx) {
            const int32_t s0 = prm.seq_idx[b * prm.T];
            seq0 = s0 < 0 ? 0 : (s0 >= prm.nseqs ? prm.nseqs - 1 : s0);
        }
        st = *(const float4*)(prm.init + (seq0 * prm.H + h) * prm.P * prm.N + 4 * e);
    }
    const int ns = prm.nseg - 1;
    const int64_t stride = (int64_t)prm.P * prm.N / 4;               // float4s per segment state
    float4* base = (float4*)(prm.seg_state + bh * ns * prm.P * prm.N) + e;
    const float* carry = prm.seg_carry + bh * ns;
    // eight segments' loads in flight before their (sequential) combine
    for (int s0 = 0; s0 < ns; s0 += 8) {
        float4 l[8];
        float c[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (s0 + k < ns) {
                l[k] = base[(s0 + k) * stride];
                c[k] = carry[s0 + k];
            }
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (s0 + k < ns) {
                // a zero carry (a sequence starts in the segment) replaces the state by a
                // select, so that an Inf or NaN state of the previous sequence does not leak
                st = c[k] == 0.f ? l[k]
                                 : make_float4(c[k] * st.x + l[k].x, c[k] * st.y + l[k].y, c[k] * st.z + l[k].z,
                                               c[k] * st.w + l[k].w);
                base[(s0 + k) * stride] = st;
            }
        }
    }
}

hipError_t launch_combine(const CombineParams& prm, hipStream_t s) {
    const int64_t threads = prm.batch * prm.H * (int64_t)prm.P * prm.N / 4;
    if (threads <= 0) return hipSuccess;
    hipLaunchKernelGGL(ssd_combine_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, prm);
    return hipGetLastError();
}
}  // namespace ssd

namespace {

using namespace ssd_host;

constexpr int64_t kMaxDim = int64_t(1) << 31;

// Tokens per kernel block.  The chunk length does not change the function (every
// chunking of the sequence gives the same outputs up to rounding), so a chunk of
// 16 or 32 tokens is evaluated in 32-token blocks and any multiple of 64 in
// 64-token blocks, with the state passed between blocks inside a chunk.
int block_len(const ssd_problem_t* p) {
    if (p->chunk_len == 16 || p->chunk_len == 32) return 32;
    if (p->chunk_len >= 64 && p->chunk_len % 64 == 0) return 64;
    return 0;
}

int64_t nblocks(const ssd_problem_t* p) {
    const int q = block_len(p);
    return q ? (p->seqlen + q - 1) / q : 0;
}

// Segments per row.  With at most 128 (row, head) items and rows of at least 16
// blocks, rows are split into
// up to 512 / items segments (256 / items where one workgroup fills a CU) that run in parallel (a local pass, a combine
// step, then the scan of every segment from its incoming state), down to 4
// blocks per segment.  (Measured on MI355X: 32 items of 256 blocks run best as
// 16 segments, or 8 with N = 256; 48 packed-sequence items of 128 blocks as 5;
// 192 items of 32 blocks run best unsplit; rows of 8 blocks ran faster unsplit.)  A function of the problem alone (no device query),
// so the workspace size is known on the host; the problem's `segments` field, when
// positive, forces the count.
struct Segs {
    int nseg, seg_blocks;
};
Segs segments(const ssd_problem_t* p) {
    const int64_t nblk = nblocks(p);
    Segs r{1, (int)(nblk > 0 ? nblk : 1)};
    if (nblk <= 1 || p->batch == 0) return r;
    int64_t S = 1;
    if (p->segments > 0) {
        S = p->segments;
    } else {
        // workgroups the scan keeps resident per CU: one where a single
        // workgroup fills the CU's registers or LDS (bf16 64-channel heads with
        // sequence ids, or with N = 256), else two
        const bool one_per_cu = p->dtype == SSD_DTYPE_BF16 && p->headdim == 64 &&
                                (p->nseqs != p->batch || p->dstate == 256);
        const int64_t slots = (one_per_cu ? 1 : 2) * 256;
        const int64_t units = p->batch * p->nheads;
        // (rows under 16 blocks stay whole: the local pass and the combine cost
        // more than the shorter walk saves)
        if (units <= 128 && nblk >= 16) S = std::min<int64_t>(slots / units, nblk / 4);
    }
    S = std::max<int64_t>(1, std::min<int64_t>(S, nblk));
    const int64_t sb = (nblk + S - 1) / S;
    r.seg_blocks = (int)sb;
    r.nseg = (int)((nblk + sb - 1) / sb);
    return r;
}

// Workspace bytes the forward pass needs: for a row split into S segments, the
// S-1 segment states (fp32 P x N per row and head) and their carried decays.
struct WsLayout {
    int64_t state_bytes, carry_off, total;
};
WsLayout ws_layout(const ssd_problem_t* p) {
    const Segs sg = segments(p);
    const int64_t n = p->batch * p->nheads * (sg.nseg - 1);
    WsLayout l;
    l.state_bytes = align256(n * p->headdim * p->dstate * 4);
    l.carry_off = l.state_bytes;
    l.total = n > 0 ? l.state_bytes + align256(n * 4) : 0;
    return l;
}
int64_t workspace_bytes(const ssd_problem_t* p) { return ws_layout(p).total; }

// 16-channel slices per scan workgroup.  One head (P / 16) by default.  With
// between 256 and 320 (row, head) items of 64 channels (bf16, no sequence ids,
// unsplit rows), five slices per workgroup spread the items evenly over 256
// workgroups (one per compute unit) instead of leaving some units with two
// heads; the slices of a workgroup must then lie in one B/C group.
int slices_per_workgroup(const ssd_problem_t* p, bool seq, int nseg) {
    const int npt = (int)(p->headdim / 16);
    const int64_t items = p->batch * p->nheads;
    if (p->dtype == SSD_DTYPE_BF16 && p->headdim == 64 && !seq && nseg == 1 && items > 256 && items <= 320 &&
        ((p->nheads / p->ngroups) * npt) % (npt + 1) == 0)
        return npt + 1;
    return npt;
}

// static_ws: the workspace is the library's own scratch array (ssd_forward_noalloc),
// which no caller buffer can overlap; ws and ws_bytes are then ignored.
int check_args(const ssd_problem_t* p, const void* x, const float* dt, const float* dt_bias, const float* A_log,
               const void* B,
               const void* C, const float* D, const float* init, const int32_t* seq_idx, const float* y,
               const float* fin, const void* ws, size_t ws_bytes, bool static_ws = false) {
    const int v = ssd_validate(p);
    if (v != SSD_OK) return v;
    const bool empty_tokens = p->batch == 0 || p->seqlen == 0;
    if (!A_log) return SSD_ERR_NULL_POINTER;
    const int64_t wsb = static_ws ? 0 : workspace_bytes(p);
    if (static_ws) {
        ws = nullptr;
        ws_bytes = 0;
    }
    if (!empty_tokens && (!x || !dt || !B || !C || !y)) return SSD_ERR_NULL_POINTER;
    if (wsb > 0 && !ws) return SSD_ERR_WORKSPACE;
    if (!seq_idx && p->nseqs != p->batch) return SSD_ERR_BAD_SHAPE;
    if (seq_idx && !empty_tokens && p->nseqs < 1) return SSD_ERR_BAD_SHAPE;   // ids need a sequence to name
    if (misaligned(x, 16) || misaligned(B, 16) || misaligned(C, 16) || misaligned(y, 16) || misaligned(dt, 4) ||
        misaligned(A_log, 4) || misaligned(dt_bias, 4) ||
        misaligned(D, 4) || misaligned(init, 16) || misaligned(fin, 16) || misaligned(seq_idx, 4) ||
        misaligned(ws, 256))
        return SSD_ERR_ALIGNMENT;
    if (static_cast<int64_t>(ws_bytes) < wsb) return SSD_ERR_WORKSPACE;
    const Sizes s = sizes(p);
    const int64_t hb = p->nheads * 4;
    // outputs must not overlap any input, the workspace or each other
    const void* in_ptr[] = {x, dt, A_log, B, C, D, seq_idx, ws, dt_bias};
    const int64_t in_sz[] = {s.x, s.dt, hb, s.bc, s.bc, hb, s.seq, wsb, hb};
    for (int i = 0; i < 9; ++i) {
        if (overlap(y, s.y, in_ptr[i], in_sz[i])) return SSD_ERR_ALIAS;
        if (overlap(fin, s.state, in_ptr[i], in_sz[i])) return SSD_ERR_ALIAS;
    }
    if (overlap(y, s.y, init, s.state) || overlap(y, s.y, fin, s.state)) return SSD_ERR_ALIAS;
    // final_state may be init_state itself (in-place carry), but not a shifted overlap
    if (fin && init && fin != init && overlap(fin, s.state, init, s.state)) return SSD_ERR_ALIAS;
    // In-place carry is safe only where every state element is read and then
    // written by one and the same wave: rows scanned in one piece and without
    // sequence ids.  With sequence ids, a sequence that starts and ends inside
    // one block has its initial state read over all N by both waves of a slice
    // while each writes its half of the final state; with rows split into
    // segments, a later segment's workgroup writes the final state of a
    // sequence whose initial state an earlier segment has yet to read.
    if (fin && fin == init && (seq_idx || segments(p).nseg > 1)) return SSD_ERR_ALIAS;
    return SSD_OK;
}

// ---- the allocation-free entry point's scratch: a file-scope device array that
// each GPU holds for the life of the process.  Host code never uses the array's
// name as an address (on the host it is only a stand-in for the symbol): the
// device address of each GPU's copy comes from hipGetSymbolAddress, taken once
// per device with that device current, and is kept here.
constexpr int64_t kScratchBytes = int64_t(SSD_NOALLOC_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the device that `stream` belongs to (the
// current device for the NULL stream).
int scratch_address(hipStream_t stream, void** out) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return SSD_ERR_HIP;
    int dev = cur;
    if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return SSD_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return SSD_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return SSD_ERR_HIP;
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (dev != cur) (void)hipSetDevice(cur);
        if (e != hipSuccess || !ptr || misaligned(ptr, 256)) return SSD_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SSD_OK;
}

int launch_scan(const ssd_problem_t* p, const void* x, const float* dt, const float* dt_bias, const float* A_log,
                const void* B,
                const void* C, const float* D, const float* init, const int32_t* seq_idx, float* y, float* fin,
                void* ws, hipStream_t stream) {
    const int q = block_len(p);
    const Segs sg = segments(p);
    const WsLayout wl = ws_layout(p);
    ssd::ScanParams prm;
    prm.x = x;
    prm.dt = dt;
    prm.A_log = A_log;
    prm.D = D;
    prm.init = init;
    prm.seq_idx = seq_idx;
    prm.y = y;
    prm.fin = fin;
    prm.B = B;
    prm.C = C;
    prm.batch = p->batch;
    prm.T = p->seqlen;
    prm.H = p->nheads;
    prm.G = p->ngroups;
    prm.nseqs = p->nseqs;
    prm.nblk = static_cast<int>(nblocks(p));
    prm.dt_bias = dt_bias;
    prm.dt_softplus = (p->flags & SSD_FLAG_DT_SOFTPLUS) ? 1 : 0;
    prm.x_scale = x_scale_of(p);
    prm.seg_blocks = sg.seg_blocks;
    prm.nseg = sg.nseg;
    prm.seg_state = sg.nseg > 1 ? static_cast<float*>(ws) : nullptr;
    prm.seg_carry = sg.nseg > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + wl.carry_off) : nullptr;
    const int64_t rows = p->batch * p->nheads;
    if (rows == 0) return SSD_OK;
    if (p->seqlen == 0 && (seq_idx || !fin)) return SSD_OK;   // no token, no sequence to hand out
    const bool seq = seq_idx != nullptr, xscale = prm.x_scale != 0;
    const int P = (int)p->headdim, N = (int)p->dstate;
    const int npt = P / 16;
    const int spw = slices_per_workgroup(p, seq, sg.nseg);
    auto scan = [&](bool local, int spw, int64_t grid) {
        return p->dtype == SSD_DTYPE_BF16 ? ssd::launch_scan_bf16(P, N, q, seq, xscale, local, spw, prm, grid, stream)
                                          : ssd::launch_scan_f32(P, N, q, seq, xscale, local, spw, prm, grid, stream);
    };

    hipError_t e = hipSuccess;
    if (sg.nseg > 1) {
        e = scan(true, spw, p->batch * (p->nheads * npt / spw) * (sg.nseg - 1));
        if (e == hipSuccess) {
            ssd::CombineParams cp;
            cp.init = init;
            cp.seq_idx = seq_idx;
            cp.seg_state = prm.seg_state;
            cp.seg_carry = prm.seg_carry;
            cp.batch = p->batch;
            cp.T = p->seqlen;
            cp.H = p->nheads;
            cp.nseqs = p->nseqs;
            cp.P = P;
            cp.N = N;
            cp.nseg = sg.nseg;
            e = ssd::launch_combine(cp, stream);
        }
    }
    if (e == hipSuccess) e = scan(false, spw, p->batch * (p->nheads * npt / spw) * sg.nseg);
    if (log_enabled())
        std::fprintf(stderr, "[ssd] scan dtype=%d P=%d N=%d QB=%d rows=%lld segments=%d x %d blocks, %d slices/wg -> %s\n",
                     p->dtype, P, N, q, (long long)rows, sg.nseg, sg.seg_blocks, spw, hipGetErrorString(e));
    return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

}  // namespace

extern "C" {

int ssd_validate(const ssd_problem_t* p) {
    if (!p) return SSD_ERR_NULL_POINTER;
    if (p->batch < 0 || p->seqlen < 0 || p->nheads <= 0 || p->headdim <= 0 || p->dstate <= 0 || p->ngroups <= 0 ||
        p->nseqs < 0)
        return SSD_ERR_BAD_SHAPE;
    if (p->batch >= kMaxDim || p->seqlen >= kMaxDim || p->nheads >= kMaxDim || p->nseqs >= kMaxDim)
        return SSD_ERR_BAD_SHAPE;
    if (p->nheads % p->ngroups != 0) return SSD_ERR_BAD_SHAPE;
    if (p->chunk_len <= 0 || p->segments < 0) return SSD_ERR_BAD_SHAPE;
    if (p->reserved != 0) return SSD_ERR_UNSUPPORTED;
    if (p->dtype != SSD_DTYPE_BF16 && p->dtype != SSD_DTYPE_F32) return SSD_ERR_UNSUPPORTED;
    if (p->flags & ~uint32_t(SSD_FLAG_DT_SCALES_X | SSD_FLAG_DT_SOFTPLUS | SSD_FLAG_ZOH)) return SSD_ERR_UNSUPPORTED;
    if ((p->flags & SSD_FLAG_DT_SCALES_X) && (p->flags & SSD_FLAG_ZOH)) return SSD_ERR_UNSUPPORTED;
    const int q = block_len(p);
    if (!q) return SSD_ERR_UNSUPPORTED;
    if (p->headdim > 4096 || p->dstate > 4096) return SSD_ERR_UNSUPPORTED;
    const int P = (int)p->headdim, N = (int)p->dstate;
    const bool ok = p->dtype == SSD_DTYPE_BF16 ? ssd::supported_bf16(P, N, q) : ssd::supported_f32(P, N, q);
    if (!ok) return SSD_ERR_UNSUPPORTED;
    // element counts must stay far from int64 overflow
    const double elems = double(p->batch) * double(p->seqlen) * double(p->nheads) * double(p->headdim);
    const double states = double(p->nseqs) * double(p->nheads) * double(p->headdim) * double(p->dstate);
    if (elems > 4e18 || states > 4e18) return SSD_ERR_BAD_SHAPE;
    if (double(p->batch) * double(p->nheads) >= 2147483647.0) return SSD_ERR_BAD_SHAPE;   // grid size
    // the kernels address one block of q tokens with 32-bit byte offsets
    if (double(q) * double(p->nheads) * double(p->headdim) * 4.0 >= 2147483647.0 ||
        double(q) * double(p->ngroups) * double(p->dstate) * 4.0 >= 2147483647.0)
        return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

size_t ssd_workspace_size(const ssd_problem_t* p) {
    if (ssd_validate(p) != SSD_OK) return 0;
    return static_cast<size_t>(workspace_bytes(p));
}

int ssd_forward(const ssd_problem_t* p, const void* x, const float* dt, const float* dt_bias, const float* A_log,
                const void* B,
                const void* C, const float* D, const float* init_state, const int32_t* seq_idx, float* y,
                float* final_state, void* workspace, size_t workspace_bytes, void* stream) {
    const int v = check_args(p, x, dt, dt_bias, A_log, B, C, D, init_state, seq_idx, y, final_state, workspace,
                             workspace_bytes);
    if (v != SSD_OK) return v;
    const int d = check_device();
    if (d != SSD_OK) return d;
    return launch_scan(p, x, dt, dt_bias, A_log, B, C, D, init_state, seq_idx, y, final_state, workspace,
                       static_cast<hipStream_t>(stream));
}

int ssd_forward_noalloc(const ssd_problem_t* p, const void* x, const float* dt, const float* dt_bias,
                        const float* A_log, const void* B, const void* C, const float* D, const float* init_state,
                        const int32_t* seq_idx, float* y, float* final_state, void* stream) {
    const int v = check_args(p, x, dt, dt_bias, A_log, B, C, D, init_state, seq_idx, y, final_state, nullptr, 0,
                             /*static_ws=*/true);
    if (v != SSD_OK) return v;
    if (workspace_bytes(p) > kScratchBytes) return SSD_ERR_SCRATCH;
    const int d = check_device();
    if (d != SSD_OK) return d;
    hipStream_t st = static_cast<hipStream_t>(stream);
    void* ws = nullptr;
    if (workspace_bytes(p) > 0) {
        const int r = scratch_address(st, &ws);
        if (r != SSD_OK) return r;
    }
    return launch_scan(p, x, dt, dt_bias, A_log, B, C, D, init_state, seq_idx, y, final_state, ws, st);
}

size_t ssd_noalloc_scratch_bytes(void) { return static_cast<size_t>(kScratchBytes); }

int ssd_step(const ssd_problem_t* p, const void* x, const float* dt, const float* dt_bias, const float* A_log,
             const void* B,
             const void* C, const float* D, float* state, float* y, void* stream) {
    if (!p) return SSD_ERR_NULL_POINTER;
    if (p->seqlen != 1 || p->nseqs != p->batch) return SSD_ERR_BAD_SHAPE;
    const int v = ssd_validate(p);
    if (v != SSD_OK) return v;
    if (!A_log) return SSD_ERR_NULL_POINTER;
    if (p->batch > 0 && (!x || !dt || !B || !C || !state || !y)) return SSD_ERR_NULL_POINTER;
    if (misaligned(x, 16) || misaligned(B, 16) || misaligned(C, 16) || misaligned(state, 16) ||
        misaligned(y, 4) || misaligned(dt, 4) || misaligned(A_log, 4) || misaligned(D, 4) || misaligned(dt_bias, 4))
        return SSD_ERR_ALIGNMENT;
    const Sizes s = sizes(p);
    const int64_t hb = p->nheads * 4;
    const void* in_ptr[] = {x, dt, A_log, B, C, D, dt_bias};
    const int64_t in_sz[] = {s.x, s.dt, hb, s.bc, s.bc, hb, hb};
    for (int i = 0; i < 7; ++i)
        if (overlap(y, s.y, in_ptr[i], in_sz[i]) || overlap(state, s.state, in_ptr[i], in_sz[i])) return SSD_ERR_ALIAS;
    if (overlap(y, s.y, state, s.state)) return SSD_ERR_ALIAS;
    const int d = check_device();
    if (d != SSD_OK) return d;
    ssd::StepParams prm;
    prm.x = x;
    prm.dt = dt;
    prm.A_log = A_log;
    prm.B = B;
    prm.C = C;
    prm.D = D;
    prm.state = state;
    prm.y = y;
    prm.batch = p->batch;
    prm.H = p->nheads;
    prm.G = p->ngroups;
    prm.dt_bias = dt_bias;
    prm.dt_softplus = (p->flags & SSD_FLAG_DT_SOFTPLUS) ? 1 : 0;
    prm.x_scale = x_scale_of(p);
    const int64_t grid = p->batch * p->nheads;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t e = p->dtype == SSD_DTYPE_BF16
                             ? ssd::launch_step_bf16((int)p->headdim, (int)p->dstate, prm, grid, st)
                             : ssd::launch_step_f32((int)p->headdim, (int)p->dstate, prm, grid, st);
    if (log_enabled())
        std::fprintf(stderr, "[ssd] step dtype=%d P=%lld N=%lld grid=%lld -> %s\n", p->dtype, (long long)p->headdim,
                     (long long)p->dstate, (long long)grid, hipGetErrorString(e));
    return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

const char* ssd_strerror(int status) {
    switch (status) {
        case SSD_OK: return "success";
        case SSD_ERR_NULL_POINTER: return "a required pointer is NULL";
        case SSD_ERR_BAD_SHAPE: return "invalid problem shape (negative size, nheads % ngroups != 0, or nseqs inconsistent)";
        case SSD_ERR_UNSUPPORTED: return "unsupported dtype, headdim, dstate, chunk_len or flags";
        case SSD_ERR_ALIGNMENT: return "a tensor pointer is misaligned (tensors need 16 bytes, the workspace 256)";
        case SSD_ERR_WORKSPACE: return "workspace missing or smaller than ssd_workspace_size()";
        case SSD_ERR_ALIAS: return "an output buffer overlaps an input, the workspace or the other output";
        case SSD_ERR_HIP: return "a HIP runtime call or kernel launch failed";
        case SSD_ERR_NO_DEVICE: return "no HIP device available";
        case SSD_ERR_SCRATCH:
            return "the problem needs more scratch than ssd_forward_noalloc's static buffer holds "
                   "(ssd_workspace_size() > ssd_noalloc_scratch_bytes()); use ssd_forward with a workspace";
        default: return "unknown ssd status code";
    }
}

int ssd_version(void) { return SSD_ABI_VERSION; }

}  // extern "C"
