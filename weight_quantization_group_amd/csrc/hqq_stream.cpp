// hqq_stream.cpp -- hqq_quantize_streamed: the solve over weights that live
// in host memory, for models larger than the device's memory (lnwmold.com
// HQQ guide section 6.3: big models are quantized a batch of layers at a
// time).
//
// The weights cross PCIe exactly once.  They are cut into chunks of whole
// row blocks that fit half of a caller-provided device staging buffer; chunk
// c is copied into half c % 2 on the copy stream while the solve of chunk
// c - 1 runs on the compute stream from the other half.  Events order the two
// streams: the first copies wait for all work enqueued on the compute stream
// before the call (an earlier call's solves may still read the staging
// buffer), a solve waits for its chunk's copy, and a copy into a half waits
// for the solve that last read it.  Each chunk is one batched solve launch
// (up to 48 row blocks), so results are identical to hqq_quantize on device
// copies of the weights.
#include "hqq.h"
#include "hqq_internal.h"

#include <stdint.h>

#include <mutex>
#include <vector>

namespace {

int64_t gcd64(int64_t a, int64_t b) { return b == 0 ? a : gcd64(b, a % b); }
int64_t lcm64(int64_t a, int64_t b) { return a / gcd64(a, b) * b; }

// Rows per block unit: whole groups and whole packed words along the group
// axis, and 16-byte aligned output offsets at every block start.
int64_t row_unit(int64_t cols, int nbits, int gs, int axis)
{
    const int64_t C = hqq::codes_per_word(nbits);
    auto align_rows = [](int64_t row_bytes) { return 16 / gcd64(16, row_bytes); };
    if (axis == 1) {
        const int64_t wpl = (cols + C - 1) / C;
        return lcm64(align_rows(wpl * 4), align_rows(cols / gs * 4));
    }
    // axis 0: a block of r rows starts r / C word rows and r / gs meta rows in
    const int64_t a = align_rows(cols * 4);
    return lcm64(lcm64(gs, C), lcm64(C * a, (int64_t)gs * a));
}

struct Piece {
    int t;           // tensor index
    int64_t r0, nr;  // row block
};

// The five events that order the copy and compute streams of one call.
struct EventSet {
    hipEvent_t copied[2] = {nullptr, nullptr}, done[2] = {nullptr, nullptr};
    hipEvent_t entry = nullptr;
    bool create()
    {
        bool ok = hipEventCreateWithFlags(&entry, hipEventDisableTiming) == hipSuccess;
        for (int b = 0; b < 2; ++b)
            ok = ok && hipEventCreateWithFlags(&copied[b], hipEventDisableTiming) == hipSuccess &&
                 hipEventCreateWithFlags(&done[b], hipEventDisableTiming) == hipSuccess;
        return ok;
    }
};

// An EventSet created for one call and released at its end.
struct Events : EventSet {
    ~Events()
    {
        // an event destroyed while still pending is released when it completes
        if (entry)
            (void)hipEventDestroy(entry);
        for (int b = 0; b < 2; ++b) {
            if (copied[b])
                (void)hipEventDestroy(copied[b]);
            if (done[b])
                (void)hipEventDestroy(done[b]);
        }
    }
};

// The staging of hqq_quantize_streamed_static: a file-scope device array.
// Host code uses only its per-device address from hipGetSymbolAddress (the
// array's name in host code is a host-side stand-in, not a device address).
// Nothing in it needs to start at zero: every byte a solve reads was copied
// in by the same call first.
constexpr int64_t kStaticStaging = HQQ_STATIC_STAGING_BYTES;
__device__ __align__(256) uint8_t scratch[kStaticStaging];

// Per device: the array's address there and the call's five events, set up
// at the first call with that device current and kept to the end of the
// process.
constexpr int kMaxDevices = 64;
struct StaticDevice {
    bool ready = false;
    void *ptr = nullptr;
    EventSet ev;
};
StaticDevice g_static[kMaxDevices];
std::mutex g_static_mu;

StaticDevice *static_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_static_mu);
    StaticDevice &d = g_static[dev];
    if (!d.ready) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return nullptr;
        EventSet ev;
        if (!ev.create())
            return nullptr;
        d.ptr = p;
        d.ev = ev;
        d.ready = true;
    }
    return &d;
}

// The streamed solve.  use_static = false: through the caller's staging
// buffer, with call_events created here for the call (after every argument
// check; the caller's Events releases them); a block unit that does not fit
// half of the buffer returns HQQ_EINVAL_SHAPE.  use_static = true: through
// the static array and the device's kept events, set up (after every
// argument check) at the first call on the current device; a block unit too
// large for it returns HQQ_ESCRATCH.
int streamed(const hqq_host_tensor *tensors, int n, int nbits, int group_size, int axis, int iters, float p,
             float beta0, float kappa, void *staging, int64_t staging_bytes, void *copy_stream,
             void *compute_stream, Events *call_events, bool use_static)
{
    const int too_big = use_static ? HQQ_ESCRATCH : HQQ_EINVAL_SHAPE;
    if (use_static)
        staging_bytes = kStaticStaging;
    if (n < 0)
        return HQQ_EINVAL_SHAPE;
    if (n > 0 && !tensors)
        return HQQ_EINVAL_PTR;
    if (const int st = hqq::check_params(iters, p, beta0, kappa))
        return st;
    if (n == 0)
        return HQQ_OK;
    if (!use_static && (!staging || ((uintptr_t)staging & 15u) != 0))
        return HQQ_EINVAL_PTR;
    // the static array is 256-byte aligned: any aligned address stands in for
    // it in the descriptor checks below
    const void *check_w = use_static ? reinterpret_cast<const void *>(uintptr_t(256)) : staging;
    // two halves of the staging buffer, 256-byte multiples (both aligned)
    const int64_t half = staging_bytes > 0 ? (staging_bytes / 2) / 256 * 256 : 0;

    // every descriptor is checked before anything is enqueued, as the
    // resident call would check it (staging stands in for W), and its block
    // unit must fit a half
    for (int i = 0; i < n; ++i) {
        const hqq_host_tensor &h = tensors[i];
        if (!h.W)
            return HQQ_EINVAL_PTR;
        const hqq_tensor d{reinterpret_cast<const uint16_t *>(check_w), h.rows, h.cols, h.packed,
                           h.scale, h.zero};
        if (const int st = hqq::check_tensor(d, nbits, group_size, axis))
            return st;
        const int64_t unit = row_unit(h.cols, nbits, group_size, axis);
        if (unit * h.cols * 2 > half)
            return too_big;
    }

    // chunks: consecutive row blocks (of one or more tensors) that fill a half
    std::vector<std::vector<Piece>> chunks(1);
    int64_t used = 0;
    for (int i = 0; i < n; ++i) {
        const hqq_host_tensor &h = tensors[i];
        const int64_t unit = row_unit(h.cols, nbits, group_size, axis);
        const int64_t row_bytes = h.cols * 2;
        int64_t r0 = 0;
        while (r0 < h.rows) {
            // room left in this chunk, in whole units (rounded so the next
            // piece also starts 256-byte aligned in the half)
            int64_t room = (half - used) / row_bytes / unit * unit;
            if (room <= 0 || (int)chunks.back().size() == hqq::kMaxBatch) {
                chunks.emplace_back();
                used = 0;
                continue;
            }
            const int64_t nr = h.rows - r0 < room ? h.rows - r0 : room;
            chunks.back().push_back(Piece{i, r0, nr});
            used += (nr * row_bytes + 255) / 256 * 256;
            r0 += nr;
        }
    }

    const hipStream_t cs = (hipStream_t)copy_stream, ks = (hipStream_t)compute_stream;
    EventSet *evs = call_events;
    if (use_static) {
        StaticDevice *d = static_device();
        if (!d)
            return HQQ_EHIP;
        staging = d->ptr;
        evs = &d->ev;
    } else if (!call_events || !call_events->create()) {
        return HQQ_EHIP;
    }
    EventSet &ev = *evs;
    // the staging buffer may still be read by solves enqueued on the compute
    // stream before this call: the copies start after them
    if (hipEventRecord(ev.entry, ks) != hipSuccess || hipStreamWaitEvent(cs, ev.entry, 0) != hipSuccess)
        return HQQ_EHIP;
    const int64_t C = hqq::codes_per_word(nbits);
    for (size_t c = 0; c < chunks.size(); ++c) {
        const int b = (int)(c & 1);
        char *buf = reinterpret_cast<char *>(staging) + b * half;
        if (c >= 2 && hipStreamWaitEvent(cs, ev.done[b], 0) != hipSuccess)
            return HQQ_EHIP;
        hqq_tensor batch[hqq::kMaxBatch];
        int64_t off = 0;
        for (size_t j = 0; j < chunks[c].size(); ++j) {
            const Piece &pc = chunks[c][j];
            const hqq_host_tensor &h = tensors[pc.t];
            const int64_t bytes = pc.nr * h.cols * 2;
            if (hipMemcpyAsync(buf + off, h.W + pc.r0 * h.cols, (size_t)bytes, hipMemcpyHostToDevice,
                               cs) != hipSuccess)
                return HQQ_EHIP;
            // outputs of the row block: rows r0 .. r0 + nr of the resident layout
            int64_t wofs, mofs;
            if (axis == 1) {
                wofs = pc.r0 * ((h.cols + C - 1) / C);
                mofs = pc.r0 * (h.cols / group_size);
            } else {
                wofs = pc.r0 / C * h.cols;
                mofs = pc.r0 / group_size * h.cols;
            }
            batch[j] = hqq_tensor{reinterpret_cast<const uint16_t *>(buf + off), pc.nr, h.cols,
                                  h.packed + wofs, h.scale + mofs, h.zero + mofs};
            off += (bytes + 255) / 256 * 256;
        }
        if (hipEventRecord(ev.copied[b], cs) != hipSuccess || hipStreamWaitEvent(ks, ev.copied[b], 0) != hipSuccess)
            return HQQ_EHIP;
        const int st = hqq_quantize_batch(batch, (int)chunks[c].size(), nbits, group_size, axis, iters, p,
                                          beta0, kappa, ks);
        if (st)
            return st;
        if (hipEventRecord(ev.done[b], ks) != hipSuccess)
            return HQQ_EHIP;
    }
    return HQQ_OK;
}

}  // namespace

extern "C" {

int hqq_quantize_streamed(const hqq_host_tensor *tensors, int n, int nbits, int group_size, int axis,
                          int iters, float p, float beta0, float kappa, void *staging,
                          int64_t staging_bytes, void *copy_stream, void *compute_stream)
{
    Events ev;
    return streamed(tensors, n, nbits, group_size, axis, iters, p, beta0, kappa, staging, staging_bytes,
                    copy_stream, compute_stream, &ev, false);
}

int hqq_quantize_streamed_static(const hqq_host_tensor *tensors, int n, int nbits, int group_size, int axis,
                                 int iters, float p, float beta0, float kappa, void *copy_stream,
                                 void *compute_stream)
{
    return streamed(tensors, n, nbits, group_size, axis, iters, p, beta0, kappa, nullptr, 0, copy_stream,
                    compute_stream, nullptr, true);
}

}  // extern "C"
