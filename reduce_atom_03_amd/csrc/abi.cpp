// abi.cpp -- the extern "C" entry points of libatom (declared in atom.h).
//
// Each call validates and plans on the host first (plan.cpp: no HIP call
// before an argument is known good), then launches the planned kernel on
// the caller's stream. The SNAC workspace is allocated per device on first
// use and kept until the process ends.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "launch.hpp"
#include "plan.hpp"

namespace atom {
namespace {

std::mutex g_ws_mutex;
Workspace g_ws[kMaxDevices];
thread_local hipError_t t_last_hip = hipSuccess;   // detail of this thread's last ATOM_ERR_HIP

atom_status hip_status(hipError_t e)
{
    if (e == hipSuccess)
        return ATOM_OK;
    t_last_hip = e;
    return ATOM_ERR_HIP;
}

// Rings replaced by a larger one. They are never freed: a HIP graph captured
// earlier keeps the address of the ring it was captured with, and work still
// in flight on any stream may use it. Rings grow at least twofold, so the
// retired ones together are smaller than the current one.
std::vector<char*> g_retired_rings;

// True when `stream` is being captured into a HIP graph (allocation is not
// allowed then; the caller is told to make one eager call first).
atom_status capturing(hipStream_t stream, bool* yes)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipError_t e = hipStreamIsCapturing(stream, &cs); e != hipSuccess)
        return hip_status(e);
    *yes = cs != hipStreamCaptureStatusNone;
    return ATOM_OK;
}

// The workspace of the current device, with a ring of at least ring_bytes.
atom_status workspace(int64_t ring_bytes, hipStream_t stream, Workspace** out)
{
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess)
        return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices)
        return ATOM_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace& ws = g_ws[dev];
    if (!ws.counts || ws.ring_bytes < ring_bytes) {
        bool cap = false;
        if (atom_status st = capturing(stream, &cap); st != ATOM_OK)
            return st;
        if (cap)
            return ATOM_ERR_UNSUPPORTED;
    }
    if (!ws.counts) {
        int khz = 0;
        if (hipError_t e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
            e != hipSuccess)
            return hip_status(e);
        if (khz <= 0)
            return ATOM_ERR_UNSUPPORTED;
        ws.wall_khz = khz;
        // counts[kMaxSlots] (each slot's count on its own 256-byte line),
        // then the ticket, the error word and the finished-workgroup count
        // on lines of their own, then the tagged ring of small calls. All
        // start at zero; every staged kernel leaves the flags at zero (the
        // error word excepted) and the tagged pairs it consumed cleared.
        char* flags = nullptr;
        const size_t line = kFlagStride * sizeof(unsigned long long);
        const size_t fbytes = (kMaxSlots + 3) * line + kTagBytes;
        if (hipMalloc(&flags, fbytes) != hipSuccess)
            return ATOM_ERR_NOMEM;
        if (hipError_t e = hipMemset(flags, 0, fbytes); e != hipSuccess) {
            (void)hipFree(flags);
            return hip_status(e);
        }
        ws.counts = reinterpret_cast<unsigned long long*>(flags);
        ws.ticket = reinterpret_cast<unsigned int*>(flags + kMaxSlots * line);
        ws.error = reinterpret_cast<unsigned int*>(flags + (kMaxSlots + 1) * line);
        ws.done = reinterpret_cast<unsigned int*>(flags + (kMaxSlots + 2) * line);
        ws.tags = reinterpret_cast<unsigned long long*>(flags + (kMaxSlots + 3) * line);
    }
    if (ws.ring_bytes < ring_bytes) {
        const int64_t want = std::max(ring_bytes, 2 * ws.ring_bytes);
        char* ring = nullptr;
        if (hipMalloc(&ring, static_cast<size_t>(want)) != hipSuccess)
            return ATOM_ERR_NOMEM;
        if (ws.ring) {
            try {
                g_retired_rings.push_back(ws.ring);
            } catch (...) {             // no exception crosses the C ABI
                (void)hipFree(ring);
                return ATOM_ERR_NOMEM;
            }
        }
        ws.ring = ring;
        ws.ring_bytes = want;
    }
    *out = &ws;
    return ATOM_OK;
}

// The next staged call's sequence number on a device (never 0, the error
// word's "no timeout"): a wait that times out records it, and only waits of
// the same call give up early because of it. It is also the tag of the
// call's words on the tagged ring; *wrapped is set when the numbers start
// over, and the caller then clears that ring before the launch.
uint32_t next_seq(Workspace* ws, bool* wrapped)
{
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    *wrapped = false;
    if (++ws->seq == 0) {
        ws->seq = 1;
        *wrapped = true;
    }
    return ws->seq;
}

atom_status run(const Plan& p, void* stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    // A launch is checked with hipGetLastError, which also returns an error
    // left behind by an earlier runtime call of this thread (ours or another
    // library's); clear it so the status describes this call only.
    if (p.exec != EX_NONE)
        (void)hipGetLastError();
    switch (p.exec) {
    case EX_NONE:
        return ATOM_OK;
    case EX_REDUCE:
        e = launch_reduce(p, s);
        break;
    case EX_COPY:
        e = launch_copy(p, s);
        break;
    case EX_SNAC_COPY:
    case EX_SNAC_REDUCE: {
        Workspace* ws = nullptr;
        atom_status st = workspace(p.ring_bytes, s, &ws);
        if (st != ATOM_OK)
            return st;
        bool wrapped = false;
        const uint32_t seq = next_seq(ws, &wrapped);
        if (wrapped && (e = launch_clear_tags(*ws, s)) != hipSuccess)
            break;
        e = launch_snac(p, *ws, seq, s);
        break;
    }
    default:
        return ATOM_ERR_UNSUPPORTED;
    }
    return hip_status(e);
}

// atom_collective_noalloc: staged plans bounded by the fixed ring, launched
// on the fixed workspace; everything else as run().
atom_status run_noalloc(const Plan& p, void* stream)
{
    if (p.exec != EX_SNAC_COPY && p.exec != EX_SNAC_REDUCE)
        return run(p, stream);
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    Workspace* ws = nullptr;
    hipError_t e = hipSuccess;
    atom_status st = static_workspace(s, &ws, &e);
    if (st == ATOM_ERR_HIP)
        return hip_status(e);
    if (st != ATOM_OK)
        return st;
    return hip_status(launch_snac(p, *ws, ws->seq, s));
}

// Reads and clears one error word after the stream was synchronized.
atom_status take_error(unsigned int* err, bool* set)
{
    *set = false;
    if (!err)
        return ATOM_OK;
    unsigned int host = 0;
    if (hipError_t e = hipMemcpy(&host, err, sizeof host, hipMemcpyDeviceToHost); e != hipSuccess)
        return hip_status(e);
    if (host == 0)
        return ATOM_OK;
    const unsigned int zero = 0;
    if (hipError_t e = hipMemcpy(err, &zero, sizeof zero, hipMemcpyHostToDevice); e != hipSuccess)
        return hip_status(e);
    *set = true;
    return ATOM_OK;
}

}  // namespace
}  // namespace atom

extern "C" {

atom_status atom_copy(void* dst, const void* src, size_t bytes, void* stream)
{
    atom::Plan p;
    atom_status st = atom::plan_copy(dst, src, bytes, nullptr, &p);
    return st == ATOM_OK ? atom::run(p, stream) : st;
}

atom_status atom_reduce(void* dst, const void* const* srcs, int32_t nsrcs, int64_t count,
                        atom_dtype dtype, atom_op op, void* stream)
{
    atom::Plan p;
    atom_status st = atom::plan_reduce(dst, srcs, nsrcs, count, dtype, op, nullptr, &p);
    return st == ATOM_OK ? atom::run(p, stream) : st;
}

atom_status atom_collective(const atom_layout* in, const atom_layout* out, atom_op op,
                            const atom_config* cfg, void* stream)
{
    atom::Plan p;
    atom_status st = atom::plan_collective(in, out, op, cfg, &p);
    return st == ATOM_OK ? atom::run(p, stream) : st;
}

atom_status atom_collective_noalloc(const atom_layout* in, const atom_layout* out, atom_op op,
                                    const atom_config* cfg, void* stream)
{
    atom::Plan p;
    atom_status st = atom::plan_collective_ex(in, out, op, cfg, atom::kStaticRingBytes, &p);
    return st == ATOM_OK ? atom::run_noalloc(p, stream) : st;
}

atom_status atom_plan_query(const atom_layout* in, const atom_layout* out, atom_op op,
                            const atom_config* cfg, atom_plan_info* info)
{
    if (!info)
        return ATOM_ERR_INVALID_ARG;
    atom::Plan p;
    atom_status st = atom::plan_collective(in, out, op, cfg, &p);
    if (st == ATOM_OK)
        atom::plan_fill_info(p, info);
    return st;
}

atom_status atom_sync_status(void* stream)
{
    if (hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream)); e != hipSuccess)
        return atom::hip_status(e);
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess)
        return atom::hip_status(e);
    if (dev < 0 || dev >= atom::kMaxDevices)
        return ATOM_ERR_UNSUPPORTED;
    unsigned int* err = nullptr;
    {
        std::lock_guard<std::mutex> lock(atom::g_ws_mutex);
        err = atom::g_ws[dev].error;
    }
    bool a = false, b = false;
    if (atom_status st = atom::take_error(err, &a); st != ATOM_OK)
        return st;
    if (atom_status st = atom::take_error(atom::static_error_word(dev), &b); st != ATOM_OK)
        return st;
    return (a || b) ? ATOM_ERR_TIMEOUT : ATOM_OK;
}

int64_t atom_moe_scratch_bytes(int32_t nranks, int32_t num_experts, int32_t topk, int64_t tokens)
{
    return atom::moe_scratch_bytes(nranks, num_experts, topk, tokens);
}

atom_status atom_moe_route(const atom_moe_routing* rt, void* stream)
{
    atom::MoeRoutePlan p;
    atom_status st = atom::plan_moe_route(rt, &p);
    if (st != ATOM_OK)
        return st;
    (void)hipGetLastError();
    return atom::hip_status(atom::launch_moe_route(p, static_cast<hipStream_t>(stream)));
}

atom_status atom_moe_dispatch(const atom_moe_routing* rt, const void* const* x, void* const* out,
                              int64_t capacity_rows, int64_t row_elems, atom_dtype dtype,
                              const atom_config* cfg, void* stream)
{
    atom::MoeMovePlan p;
    atom_status st =
        atom::plan_moe_move(rt, false, x, nullptr, out, capacity_rows, row_elems, dtype, cfg, &p);
    if (st != ATOM_OK)
        return st;
    (void)hipGetLastError();
    return atom::hip_status(atom::launch_moe_move(p, false, static_cast<hipStream_t>(stream)));
}

atom_status atom_moe_combine(const atom_moe_routing* rt, const void* const* y, const float* const* weights,
                             void* const* out, int64_t capacity_rows, int64_t row_elems, atom_dtype dtype,
                             const atom_config* cfg, void* stream)
{
    atom::MoeMovePlan p;
    atom_status st =
        atom::plan_moe_move(rt, true, y, weights, out, capacity_rows, row_elems, dtype, cfg, &p);
    if (st != ATOM_OK)
        return st;
    (void)hipGetLastError();
    return atom::hip_status(atom::launch_moe_move(p, true, static_cast<hipStream_t>(stream)));
}

const char* atom_last_error(void)
{
    return atom::t_last_hip == hipSuccess ? "no HIP error" : hipGetErrorString(atom::t_last_hip);
}

int64_t atom_bdp_chunk_bytes(double bytes_per_s, double round_trip_s)
{
    return atom::bdp_chunk_bytes(bytes_per_s, round_trip_s);
}

const char* atom_status_string(atom_status s)
{
    switch (s) {
    case ATOM_OK: return "ok";
    case ATOM_ERR_INVALID_ARG: return "invalid argument";
    case ATOM_ERR_UNSUPPORTED: return "unsupported layout/op combination";
    case ATOM_ERR_HIP: return "HIP runtime error";
    case ATOM_ERR_TIMEOUT: return "SNAC wait timed out on the device";
    case ATOM_ERR_NOMEM: return "workspace allocation failed";
    case ATOM_ERR_LIMIT: return "staged call exceeds the fixed workspace of atom_collective_noalloc";
    }
    return "unknown status";
}

atom_status atom_device_clock_khz(int32_t* khz)
{
    if (!khz)
        return ATOM_ERR_INVALID_ARG;
    int dev = 0, v = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess)
        return atom::hip_status(e);
    if (hipError_t e = hipDeviceGetAttribute(&v, hipDeviceAttributeWallClockRate, dev); e != hipSuccess)
        return atom::hip_status(e);
    *khz = v;
    return ATOM_OK;
}

int32_t atom_version(void) { return (0 << 16) | 1; }

}  // extern "C"
