// zc_api.hip -- the C ABI: plans, argument checks and launch sequences.
//
// Compress (ZipCCL scribe notes, "Key idea and contribution", technique 1):
//   zc_encode          fp64 moment partials per 16,384-value block, and the
//                      codes, sign+mantissa bytes, staged escape exponents
//                      and escape counts, with each segment's previous window
//                      as the prediction (or the caller's fixed window)
//   zc_finish          the two kernels below in one launch, overlapped
//                      (segments up to 16,384 moment blocks, no raw fallback,
//                      no split event); a failed prediction is coded again
//                      chunk by chunk there
//   zc_window          per segment: variance -> window, statistics, header
//                      fields known before encoding; where the prediction
//                      failed, the segment's codes again; chunk table, sizes;
//                      with the raw fallback, the raw header where coding
//                      would not shrink the segment
//   zc_place_escapes   group table, escapes to their place (a raw segment:
//                      its values after the header)
// Decompress: zc_decode.  Decompress-reduce: zc_decode_reduce_wide (one wave
// per shard, up to 8 shards), else zc_decode_reduce (shards in turn).
// Every call enqueues on the caller's stream and returns; nothing here reads
// device memory except the two zc_read_* helpers, which synchronise.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "zc.h"
#include "zc_kernels.h"
#include "zc_plan_layout.h"

using namespace zc;

static_assert(kPlanRawFallback == ZC_PLAN_RAW_FALLBACK, "plan flag values agree");

struct zc_plan : zc::PlanLayout {  // the host layout plus its device tables
    SegDesc* d_segs = nullptr;
    ItemDesc* d_chunks = nullptr;
    ItemDesc* d_groups = nullptr;
    ItemDesc* d_pairs = nullptr;
    ItemDesc* d_witems = nullptr;
    ItemDesc* d_fitems = nullptr;
};

namespace {

// The workspace of zc_compress_static: a file-scope device array, one copy
// per GPU, held until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: host code uses only the
// address hipGetSymbolAddress returns for the current device.
constexpr uint64_t kScratchBytes = 80ull << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (set up once per device, with that
// device current), or null if the lookup failed.
void* scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();  // leave no error for the caller's next call
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

uint64_t cdiv(uint64_t a, uint64_t b) { return (a + b - 1) / b; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

uint32_t nchunks(const zc_plan* p) { return (uint32_t)p->chunks.size(); }
uint32_t ngroups(const zc_plan* p) { return (uint32_t)p->groups.size(); }
uint32_t group_grid(const zc_plan* p) { return (ngroups(p) + 3) / 4; }

zc_status launch_status() {
    return hipGetLastError() == hipSuccess ? ZC_OK : ZC_ERR_HIP;
}

zc_status check_ws(const zc_plan* p, const void* d_ws, uint64_t ws_bytes) {
    if (!d_ws || !aligned(d_ws, 256)) return ZC_ERR_INVALID_ARG;
    if (ws_bytes < p->ws.total) return ZC_ERR_CAPACITY;
    return ZC_OK;
}

// The decoders need the status words and the stand-in only.
zc_status check_dec_ws(const zc_plan* p, const void* d_ws, uint64_t ws_bytes) {
    if (!d_ws || !aligned(d_ws, 256)) return ZC_ERR_INVALID_ARG;
    if (ws_bytes < p->ws.dec_total) return ZC_ERR_CAPACITY;
    return ZC_OK;
}

template <typename T>
T* ws_ptr(const zc_plan*, void* d_ws, uint64_t off) {
    return reinterpret_cast<T*>(static_cast<uint8_t*>(d_ws) + off);
}

// ev: null, or four events recorded on the stream around the three kernels;
// fixed: null, or an event recorded once the fixed-size regions are final
zc_status compress_impl(const zc_plan* p, const void* d_in, void* d_out, uint64_t out_capacity,
                        uint64_t* d_stream_bytes, uint32_t forced_L, void* d_ws, uint64_t ws_bytes,
                        hipStream_t stream, hipEvent_t* ev = nullptr, hipEvent_t fixed = nullptr) {
    if (!p) return ZC_ERR_INVALID_ARG;
    if (p->input_elems && (!d_in || !aligned(d_in, 16))) return ZC_ERR_INVALID_ARG;
    if (!d_out || !aligned(d_out, 256) || !d_stream_bytes || !aligned(d_stream_bytes, 8))
        return ZC_ERR_INVALID_ARG;
    if (out_capacity < p->out_bytes) return ZC_ERR_CAPACITY;
    if (zc_status e = check_ws(p, d_ws, ws_bytes)) return e;

    const uint32_t nwg = (uint32_t)(p->pairs.size() / 4);
    EncodeArgs ea{};
    ea.segs = p->d_segs;
    ea.pairs = p->d_pairs;
    ea.in = static_cast<const uint16_t*>(d_in);
    ea.out = static_cast<uint8_t*>(d_out);
    ea.stats = ws_ptr<SegStat>(p, d_ws, p->ws.stats);
    ea.part.s1 = ws_ptr<double>(p, d_ws, p->ws.ps1);
    ea.part.s2 = ws_ptr<double>(p, d_ws, p->ws.ps2);
    ea.part.n = ws_ptr<uint32_t>(p, d_ws, p->ws.pn);
    ea.part.esc = ws_ptr<uint32_t>(p, d_ws, p->ws.pesc);
    ea.pred = ws_ptr<uint32_t>(p, d_ws, p->ws.pred);
    ea.done = ws_ptr<uint32_t>(p, d_ws, p->ws.done);
    ea.zero = ws_ptr<uint32_t>(p, d_ws, p->ws.zero);
    ea.staging = ws_ptr<uint8_t>(p, d_ws, p->ws.staging);
    ea.gcnt = ws_ptr<uint32_t>(p, d_ws, p->ws.gcnt);
    ea.flag = ws_ptr<uint32_t>(p, d_ws, p->ws.flag);
    ea.agg = ws_ptr<uint64_t>(p, d_ws, p->ws.agg);
    ea.fpart = ws_ptr<uint64_t>(p, d_ws, p->ws.fpart);
    ea.chunk_elems = p->chunk;
    ea.block_elems = p->block;
    ea.forced_L = forced_L;
    ea.single = p->nseg == 1;
    ea.seg0 = p->segs[0];
    if (ev && hipEventRecord(ev[0], stream) != hipSuccess) return ZC_ERR_HIP;
    if (nwg) {
        // grids of at most 256 items (4M values) take eight waves of one
        // group each, so a wave's chain is one group long (1M values:
        // compress 21.5 us against 24; 8M: even; 16M and up: slower, the
        // second group's loads no longer overlap the first's moments)
        if (forced_L) hipLaunchKernelGGL((zc_encode<false, 2>), dim3(nwg), dim3(256), 0, stream, ea);
        else if (nwg <= 256) hipLaunchKernelGGL((zc_encode<true, 1>), dim3(nwg), dim3(512), 0, stream, ea);
        else hipLaunchKernelGGL((zc_encode<true, 2>), dim3(nwg), dim3(256), 0, stream, ea);
    }
    if (ev && hipEventRecord(ev[1], stream) != hipSuccess) return ZC_ERR_HIP;
    WindowArgs wa{ea, p->d_witems, ws_ptr<SegStat>(p, d_ws, p->ws.stats), d_stream_bytes,
                  p->chunk, p->chunk / p->block, (p->flags & ZC_PLAN_RAW_FALLBACK) ? 1u : 0u};
    uint8_t* out = static_cast<uint8_t*>(d_out);
    const PlaceArgs pa{p->d_segs, p->d_chunks, out, ea.staging, ea.gcnt, ea.in, p->chunk, nchunks(p),
                       p->nseg == 1, p->segs[0]};
    if (p->merged_tail && !fixed) {
        // the window check and the placement in one launch (zc_finish.hip):
        // one window workgroup per segment, then one workgroup per chunk
        const uint32_t nwin = (uint32_t)p->fitems.size();
        const FinishArgs fa{wa, pa, p->d_fitems, nwin};
        const dim3 grid(nwin + nchunks(p));
        // groups per wave of the 4-wave placement workgroups (a chunk holds
        // 1 to 32 groups, a power of two): 1, 2, 4 or 8; waves past the
        // chunk's last group idle
        const uint32_t gpc = p->chunk / kGroup;
        const uint32_t gpw = gpc > 4 ? gpc / 4 : 1;
        auto launch = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, fa); };
        if (ea.single) {
            if (gpw == 1) launch(zc_finish<true, 1>);
            else if (gpw == 2) launch(zc_finish<true, 2>);
            else if (gpw == 4) launch(zc_finish<true, 4>);
            else launch(zc_finish<true, 8>);
        } else {
            if (gpw == 1) launch(zc_finish<false, 1>);
            else if (gpw == 2) launch(zc_finish<false, 2>);
            else if (gpw == 4) launch(zc_finish<false, 4>);
            else launch(zc_finish<false, 8>);
        }
        if (ev && (hipEventRecord(ev[2], stream) != hipSuccess || hipEventRecord(ev[3], stream) != hipSuccess))
            return ZC_ERR_HIP;
        return launch_status();
    }
    if (ea.single) hipLaunchKernelGGL(zc_window<true>, dim3((uint32_t)p->witems.size()), dim3(256), 0, stream, wa);
    else hipLaunchKernelGGL(zc_window<false>, dim3((uint32_t)p->witems.size()), dim3(256), 0, stream, wa);
    if (ev && hipEventRecord(ev[2], stream) != hipSuccess) return ZC_ERR_HIP;
    // after the window kernel: codes and sm bytes (coded again there when
    // the prediction failed), header, chunk table and sizes are final
    if (fixed && hipEventRecord(fixed, stream) != hipSuccess) return ZC_ERR_HIP;
    if (nchunks(p)) {
        const uint32_t gpc = p->chunk / kGroup;
        // placement: up to 4 waves, each with gpc / waves groups
        const uint32_t pw = gpc < 4 ? gpc : 4;
        const dim3 pblock(64 * pw);
        const dim3 pgrid(nchunks(p));  // one chunk per workgroup: latency hides across chunks
        switch (gpc / pw) {
            case 1: hipLaunchKernelGGL((zc_place_escapes<1>), pgrid, pblock, 0, stream, pa); break;
            case 2: hipLaunchKernelGGL((zc_place_escapes<2>), pgrid, pblock, 0, stream, pa); break;
            case 4: hipLaunchKernelGGL((zc_place_escapes<4>), pgrid, pblock, 0, stream, pa); break;
            default: hipLaunchKernelGGL((zc_place_escapes<8>), pgrid, pblock, 0, stream, pa); break;
        }
    }
    if (ev && hipEventRecord(ev[3], stream) != hipSuccess) return ZC_ERR_HIP;
    return launch_status();
}

}  // namespace

extern "C" {

int zc_version(void) { return 1; }

const char* zc_status_string(zc_status s) {
    switch (s) {
        case ZC_OK: return "ok";
        case ZC_ERR_INVALID_ARG: return "invalid argument";
        case ZC_ERR_CAPACITY: return "buffer too small";
        case ZC_ERR_UNSUPPORTED: return "unsupported size";
        case ZC_ERR_FORMAT: return "stream rejected";
        case ZC_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

zc_status zc_plan_create(uint32_t num_segments, const uint64_t* segment_elems, uint32_t chunk_elems,
                         zc_plan** out_plan) {
    return zc_plan_create_ex(num_segments, segment_elems, chunk_elems, 0u, out_plan);
}

zc_status zc_plan_create_ex(uint32_t num_segments, const uint64_t* segment_elems, uint32_t chunk_elems,
                            uint32_t flags, zc_plan** out_plan) {
    if (!out_plan || num_segments == 0 || !segment_elems) return ZC_ERR_INVALID_ARG;
    *out_plan = nullptr;
    if (flags & ~ZC_PLAN_RAW_FALLBACK) return ZC_ERR_INVALID_ARG;
    zc_plan* p = new (std::nothrow) zc_plan;
    if (!p) return ZC_ERR_HIP;
    if (const int e = build_layout(num_segments, segment_elems, chunk_elems, flags, *p)) {
        delete p;
        return static_cast<zc_status>(e);
    }
    const uint64_t G = p->groups.size(), K = p->chunks.size(), W = p->pairs.size();
    if (hipMalloc(&p->d_segs, sizeof(SegDesc) * p->segs.size()) != hipSuccess ||
        hipMalloc(&p->d_chunks, sizeof(ItemDesc) * (K ? K : 1)) != hipSuccess ||
        hipMalloc(&p->d_groups, sizeof(ItemDesc) * (G ? G : 1)) != hipSuccess ||
        hipMalloc(&p->d_pairs, sizeof(ItemDesc) * (W ? W : 1)) != hipSuccess ||
        hipMalloc(&p->d_witems, sizeof(ItemDesc) * p->witems.size()) != hipSuccess ||
        hipMalloc(&p->d_fitems, sizeof(ItemDesc) * p->fitems.size()) != hipSuccess ||
        hipMemcpy(p->d_fitems, p->fitems.data(), sizeof(ItemDesc) * p->fitems.size(),
                  hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(p->d_segs, p->segs.data(), sizeof(SegDesc) * p->segs.size(),
                  hipMemcpyHostToDevice) != hipSuccess ||
        (K && hipMemcpy(p->d_chunks, p->chunks.data(), sizeof(ItemDesc) * K,
                        hipMemcpyHostToDevice) != hipSuccess) ||
        (G && hipMemcpy(p->d_groups, p->groups.data(), sizeof(ItemDesc) * G,
                        hipMemcpyHostToDevice) != hipSuccess) ||
        (W && hipMemcpy(p->d_pairs, p->pairs.data(), sizeof(ItemDesc) * W,
                        hipMemcpyHostToDevice) != hipSuccess) ||
        hipMemcpy(p->d_witems, p->witems.data(), sizeof(ItemDesc) * p->witems.size(),
                  hipMemcpyHostToDevice) != hipSuccess) {
        zc_plan_destroy(p);
        return ZC_ERR_HIP;
    }
    // set-up of zc_compress_static's array on this device (a failure here is
    // reported by that call, not by the plan)
    (void)scratch_for_current_device();
    *out_plan = p;
    return ZC_OK;
}

void zc_plan_destroy(zc_plan* p) {
    if (!p) return;
    if (p->d_segs) (void)hipFree(p->d_segs);
    if (p->d_chunks) (void)hipFree(p->d_chunks);
    if (p->d_groups) (void)hipFree(p->d_groups);
    if (p->d_pairs) (void)hipFree(p->d_pairs);
    if (p->d_witems) (void)hipFree(p->d_witems);
    if (p->d_fitems) (void)hipFree(p->d_fitems);
    delete p;
}

uint32_t zc_plan_num_segments(const zc_plan* p) { return p ? p->nseg : 0; }
uint32_t zc_plan_chunk_elems(const zc_plan* p) { return p ? p->chunk : 0; }
uint32_t zc_plan_flags(const zc_plan* p) { return p ? p->flags : 0; }
uint64_t zc_plan_input_offset(const zc_plan* p, uint32_t s) {
    return p && s < p->nseg ? p->segs[s].in_off : 0;
}
uint64_t zc_plan_input_elems(const zc_plan* p) { return p ? p->input_elems : 0; }
uint64_t zc_plan_stream_offset(const zc_plan* p, uint32_t s) {
    return p && s < p->nseg ? p->segs[s].out_off : 0;
}
uint64_t zc_plan_code_offset(const zc_plan* p, uint32_t s) {
    return p && s < p->nseg ? p->segs[s].code_off : 0;
}
uint64_t zc_plan_escape_offset(const zc_plan* p, uint32_t s) {
    return p && s < p->nseg ? p->segs[s].esc_off : 0;
}
uint64_t zc_plan_max_stream_bytes(const zc_plan* p, uint32_t s) {
    return p && s < p->nseg ? p->segs[s].max_bytes : 0;
}
uint64_t zc_plan_out_bytes(const zc_plan* p) { return p ? p->out_bytes : 0; }
uint64_t zc_plan_workspace_bytes(const zc_plan* p) { return p ? p->ws.total : 0; }
uint64_t zc_plan_decode_workspace_bytes(const zc_plan* p) { return p ? p->ws.dec_total : 0; }

zc_status zc_compress(const zc_plan* p, const void* d_in, void* d_out, uint64_t out_capacity,
                      uint64_t* d_stream_bytes, void* d_ws, uint64_t ws_bytes, hipStream_t stream) {
    return compress_impl(p, d_in, d_out, out_capacity, d_stream_bytes, 0, d_ws, ws_bytes, stream);
}

zc_status zc_compress_split(const zc_plan* p, const void* d_in, void* d_out, uint64_t out_capacity,
                            uint64_t* d_stream_bytes, void* d_ws, uint64_t ws_bytes,
                            hipStream_t stream, hipEvent_t fixed_ready) {
    // a raw stream rewrites its fixed regions after the event: no split then
    if (!fixed_ready || !p || (p->flags & ZC_PLAN_RAW_FALLBACK)) return ZC_ERR_INVALID_ARG;
    return compress_impl(p, d_in, d_out, out_capacity, d_stream_bytes, 0, d_ws, ws_bytes, stream,
                         nullptr, fixed_ready);
}

zc_status zc_compress_timed(const zc_plan* p, const void* d_in, void* d_out, uint64_t out_capacity,
                            uint64_t* d_stream_bytes, void* d_ws, uint64_t ws_bytes,
                            hipStream_t stream, float* us) {
    if (!us) return ZC_ERR_INVALID_ARG;
    hipEvent_t ev[4] = {};
    zc_status st = ZC_OK;
    for (auto& e : ev)
        if (hipEventCreate(&e) != hipSuccess) st = ZC_ERR_HIP;
    if (st == ZC_OK)
        st = compress_impl(p, d_in, d_out, out_capacity, d_stream_bytes, 0, d_ws, ws_bytes, stream, ev);
    if (st == ZC_OK && hipEventSynchronize(ev[3]) != hipSuccess) st = ZC_ERR_HIP;
    for (int k = 0; st == ZC_OK && k < 3; ++k) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, ev[k], ev[k + 1]) != hipSuccess) st = ZC_ERR_HIP;
        us[k] = 1000.f * ms;
    }
    // a merged plan records its last two events back to back (no kernel
    // between them): what they read is the events' own overhead, not a
    // kernel's time
    if (st == ZC_OK && p->merged_tail) us[2] = 0.f;
    for (auto& e : ev)
        if (e) (void)hipEventDestroy(e);
    return st;
}

zc_status zc_compress_static(const zc_plan* p, const void* d_in, void* d_out, uint64_t out_capacity,
                             uint64_t* d_stream_bytes, hipStream_t stream) {
    if (!p) return ZC_ERR_INVALID_ARG;
    if (p->ws.total > kScratchBytes) return ZC_ERR_CAPACITY;  // plan too large for the array
    void* ws = scratch_for_current_device();
    if (!ws) return ZC_ERR_HIP;
    return compress_impl(p, d_in, d_out, out_capacity, d_stream_bytes, 0, ws, kScratchBytes, stream);
}

uint64_t zc_static_workspace_bytes(void) { return kScratchBytes; }

zc_status zc_compress_window(const zc_plan* p, const void* d_in, void* d_out, uint64_t out_capacity,
                             uint64_t* d_stream_bytes, uint32_t window_L, void* d_ws,
                             uint64_t ws_bytes, hipStream_t stream) {
    if (window_L < 1 || window_L > 248) return ZC_ERR_INVALID_ARG;
    return compress_impl(p, d_in, d_out, out_capacity, d_stream_bytes, window_L, d_ws, ws_bytes,
                         stream);
}

zc_status zc_decompress(const zc_plan* p, const void* d_in, uint64_t in_capacity, void* d_out,
                        void* d_ws, uint64_t ws_bytes, hipStream_t stream) {
    if (!p || !d_in || !aligned(d_in, 256)) return ZC_ERR_INVALID_ARG;
    if (p->input_elems && (!d_out || !aligned(d_out, 16))) return ZC_ERR_INVALID_ARG;
    if (zc_status e = check_dec_ws(p, d_ws, ws_bytes)) return e;
    if (!ngroups(p)) return ZC_OK;
    DecodeArgs a{};
    a.segs = p->d_segs;
    a.groups = p->d_groups;
    a.single = p->nseg == 1;
    a.seg0 = p->segs[0];
    a.in[0] = static_cast<const uint8_t*>(d_in);
    a.capacity = in_capacity;
    a.nstreams = 1;
    a.chunk_elems = p->chunk;
    a.ngroups = ngroups(p);
    a.out = static_cast<uint16_t*>(d_out);
    a.status = ws_ptr<uint32_t>(p, d_ws, p->ws.status);
    a.dummy = ws_ptr<uint8_t>(p, d_ws, p->ws.dummy);  // 2048 readable bytes
    if (a.single) hipLaunchKernelGGL(zc_decode<true>, dim3(group_grid(p)), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(zc_decode<false>, dim3(group_grid(p)), dim3(256), 0, stream, a);
    return launch_status();
}

zc_status zc_decompress_reduce(const zc_plan* p, const void* const* d_streams, uint32_t nstreams,
                               uint64_t stream_capacity, void* d_out, void* d_ws, uint64_t ws_bytes,
                               hipStream_t stream) {
    if (!p || p->nseg != 1 || !d_streams || nstreams < 1 || nstreams > kMaxStreams)
        return ZC_ERR_INVALID_ARG;
    for (uint32_t s = 0; s < nstreams; ++s)
        if (!d_streams[s] || !aligned(d_streams[s], 256)) return ZC_ERR_INVALID_ARG;
    if (p->input_elems && (!d_out || !aligned(d_out, 16))) return ZC_ERR_INVALID_ARG;
    if (zc_status e = check_dec_ws(p, d_ws, ws_bytes)) return e;
    if (!ngroups(p)) return ZC_OK;
    DecodeArgs a{};
    a.segs = p->d_segs;
    a.groups = p->d_groups;
    a.single = p->nseg == 1;
    a.seg0 = p->segs[0];
    for (uint32_t s = 0; s < nstreams; ++s) a.in[s] = static_cast<const uint8_t*>(d_streams[s]);
    a.capacity = stream_capacity;
    a.nstreams = nstreams;
    a.chunk_elems = p->chunk;
    a.ngroups = ngroups(p);
    a.out = static_cast<uint16_t*>(d_out);
    a.status = ws_ptr<uint32_t>(p, d_ws, p->ws.status);
    a.dummy = ws_ptr<uint8_t>(p, d_ws, p->ws.dummy);  // 2048 readable bytes
    if (nstreams <= 8) {  // one wave per shard, one workgroup per group
        void (*k)(DecodeArgs) = nullptr;
        switch (nstreams) {
            case 1: k = zc_decode_reduce_wide<1>; break;
            case 2: k = zc_decode_reduce_wide<2>; break;
            case 3: k = zc_decode_reduce_wide<3>; break;
            case 4: k = zc_decode_reduce_wide<4>; break;
            case 5: k = zc_decode_reduce_wide<5>; break;
            case 6: k = zc_decode_reduce_wide<6>; break;
            case 7: k = zc_decode_reduce_wide<7>; break;
            default: k = zc_decode_reduce_wide<8>; break;
        }
        hipLaunchKernelGGL(k, dim3(ngroups(p)), dim3(64 * nstreams), 0, stream, a);
    } else
        hipLaunchKernelGGL(zc_decode_reduce, dim3(group_grid(p)), dim3(256), 0, stream, a);
    return launch_status();
}

zc_status zc_read_status(const zc_plan* p, const void* d_ws, hipStream_t stream, uint32_t* host_bits) {
    if (!p || !d_ws || !host_bits) return ZC_ERR_INVALID_ARG;
    *host_bits = 0;
    if (hipStreamSynchronize(stream) != hipSuccess) return ZC_ERR_HIP;
    const uint32_t K = ngroups(p);
    if (!K) return ZC_OK;
    std::vector<uint32_t> st(K);
    if (hipMemcpy(st.data(), static_cast<const uint8_t*>(d_ws) + p->ws.status, 4ull * K,
                  hipMemcpyDeviceToHost) != hipSuccess)
        return ZC_ERR_HIP;
    uint32_t bits = 0;
    for (uint32_t v : st) bits |= v;
    *host_bits = bits;
    return bits ? ZC_ERR_FORMAT : ZC_OK;
}

zc_status zc_read_sigma(const zc_plan* p, const void* d_ws, uint32_t s, hipStream_t stream,
                        double* S1, double* S2, uint64_t* n, double* var, uint32_t* L) {
    if (!p || !d_ws || s >= p->nseg) return ZC_ERR_INVALID_ARG;
    if (hipStreamSynchronize(stream) != hipSuccess) return ZC_ERR_HIP;
    SegStat st;
    if (hipMemcpy(&st, static_cast<const uint8_t*>(d_ws) + p->ws.stats + sizeof(SegStat) * s,
                  sizeof st, hipMemcpyDeviceToHost) != hipSuccess)
        return ZC_ERR_HIP;
    if (S1) *S1 = st.s1;
    if (S2) *S2 = st.s2;
    if (n) *n = st.n;
    if (var) *var = st.var;
    if (L) *L = st.L;
    return ZC_OK;
}

zc_status zc_reduce_native(const void* const* d_shards, uint32_t nshards, uint64_t n, void* d_out,
                           hipStream_t stream) {
    if (!d_shards || nshards < 1 || nshards > kMaxStreams) return ZC_ERR_INVALID_ARG;
    if (n && (!d_out || !aligned(d_out, 16))) return ZC_ERR_INVALID_ARG;
    NativeReduceArgs a{};
    for (uint32_t s = 0; s < nshards; ++s) {
        if (n && (!d_shards[s] || !aligned(d_shards[s], 16))) return ZC_ERR_INVALID_ARG;
        a.in[s] = static_cast<const uint16_t*>(d_shards[s]);
    }
    if (!n) return ZC_OK;
    a.out = static_cast<uint16_t*>(d_out);
    a.n = n;
    // one 8-value word per thread (a grid-stride loop past 2^20 workgroups)
    const dim3 grid((uint32_t)std::min<uint64_t>(std::max<uint64_t>(1, cdiv(n / 8, 256)), 1u << 20));
    switch (nshards) {
#define ZC_NATIVE_CASE(S) \
        case S: hipLaunchKernelGGL(zc_reduce_native<S>, grid, dim3(256), 0, stream, a); break;
        ZC_NATIVE_CASE(1) ZC_NATIVE_CASE(2) ZC_NATIVE_CASE(3) ZC_NATIVE_CASE(4)
        ZC_NATIVE_CASE(5) ZC_NATIVE_CASE(6) ZC_NATIVE_CASE(7) ZC_NATIVE_CASE(8)
        ZC_NATIVE_CASE(9) ZC_NATIVE_CASE(10) ZC_NATIVE_CASE(11) ZC_NATIVE_CASE(12)
        ZC_NATIVE_CASE(13) ZC_NATIVE_CASE(14) ZC_NATIVE_CASE(15) ZC_NATIVE_CASE(16)
#undef ZC_NATIVE_CASE
    }
    return launch_status();
}

int zc_prefer_compressed(uint64_t raw_bytes, uint64_t compressed_bytes, double compress_us,
                         double decompress_us, double link_GBps, double* break_even_GBps) {
    if (break_even_GBps) *break_even_GBps = 0.0;
    if (!(link_GBps > 0.0) || !(compress_us >= 0.0) || !(decompress_us >= 0.0)) return 0;
    const double saved = (double)raw_bytes - (double)compressed_bytes;  // bytes
    const double cost_us = compress_us + decompress_us;
    if (break_even_GBps && saved > 0.0)
        *break_even_GBps = cost_us > 0.0 ? saved / (cost_us * 1e3) : INFINITY;  // bytes/us -> GB/s
    // compare the link time saved (us) with the codec's time
    return saved > 0.0 && saved / (link_GBps * 1e3) > cost_us ? 1 : 0;
}

}  // extern "C"
