// Device-side entry points of the C ABI: bind a workspace, launch the forward
// and merge kernels.  The library never allocates device memory; the caller
// provides every device buffer (the workspace included).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstdint>
#include <mutex>
#include <string>

#include "kvattn_plan.hpp"

namespace kvattn {
namespace {

// Device pointers of the plan's workspace sections at `ws` (the bound workspace,
// or the static scratch of kvattn_decode_noalloc), for forward launch `launch`
// (-1: the merge).
DevPlan resolve(const kvattn_plan_s& P, int launch, void* ws) {
    auto* base = static_cast<unsigned char*>(ws);
    const BlobHeader& h = P.header;
    DevPlan d;
    d.desc = reinterpret_cast<const int32_t*>(base + h.off_desc);
    d.list_ptr = reinterpret_cast<const int32_t*>(base + h.off_list_ptr);
    d.n_lists = P.n_lists;
    if (launch >= 0) d.list_ptr += size_t(launch) * size_t(P.n_lists) * 3;
    d.merge_rec = reinterpret_cast<const MergeRec*>(base + h.off_merge_rec);
    d.claim = reinterpret_cast<int32_t*>(base + h.off_claim);
    if (launch >= 0) d.claim += P.forward_launches[size_t(launch)].side;   // concurrent launches count apart
    d.part_ml = reinterpret_cast<float*>(base + h.off_part_ml);
    d.part_acc = reinterpret_cast<float*>(base + h.off_part_acc);
    d.arrive = P.fused_merge ? reinterpret_cast<int32_t*>(base + h.off_arrive) : nullptr;
    // < 4 GiB whenever the plan fuses its merge (the planner checks); larger arrays
    // are written with plain stores and 64-bit addresses (part_wt 0).  The
    // environment variable KVATTN_PLAIN_PARTIALS=1 takes that path at any size
    // (plans without a fused merge), so tests can check it on small batches.
    const uint64_t acc_bytes = uint64_t(P.n_slots) * uint64_t(h.head_dim) * 4;
    d.part_ml_bytes = uint32_t(std::min<uint64_t>(uint64_t(P.n_slots) * 8, 0xFFFFFFF0u));
    d.part_acc_bytes = uint32_t(std::min<uint64_t>(acc_bytes, 0xFFFFFFF0u));
    const char* plain = std::getenv("KVATTN_PLAIN_PARTIALS");
    const bool force_plain = plain && plain[0] == '1' && !P.fused_merge;
    d.part_wt = acc_bytes <= 0xFFFFFFF0u && !force_plain ? 1 : 0;
    d.has_split = P.has_split ? 1 : 0;
    return d;
}

Dims dims(const kvattn_plan_s& P) {
    Dims d;
    d.num_q_heads = P.shape.num_q_heads;
    d.num_kv_heads = P.shape.num_kv_heads;
    d.head_dim = P.shape.head_dim;
    d.group = P.shape.num_q_heads / P.shape.num_kv_heads;
    d.scale_log2 = float(double(P.scale) * 1.4426950408889634);
    return d;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Host wait for the event recorded after a plan's last upload copy.
void wait_upload_event(void* event) { (void)hipEventSynchronize(static_cast<hipEvent_t>(event)); }

kvattn_status check_bound(kvattn_plan_t plan) {
    if (!plan) return set_error(KVATTN_EINVAL, "plan is NULL");
    if (!plan->dev_ws) return set_error(KVATTN_ESTATE, "no device workspace bound: call kvattn_plan_upload first");
    return KVATTN_OK;
}

kvattn_status run_forward(const void* q, const void* k, const void* v, kvattn_plan_t plan, float* out,
                          void* stream, void* side_stream = nullptr, void* ws = nullptr) {
    if (!ws) ws = plan->dev_ws;
    if (!q || !k || !v || !out) return set_error(KVATTN_EINVAL, "q, k_cache, v_cache or out is NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return set_error(KVATTN_EINVAL, "q, k_cache, v_cache and out must be 16-byte aligned");
    const Dims d = dims(*plan);
    // Each launch drains its queues of MFMA and VALU tasks; launches (normally
    // one) follow each other on `stream`.
    for (const Launch& L : plan->forward_launches) {
        const DevPlan dp = resolve(*plan, L.index, ws);
        void* s = L.side && side_stream ? side_stream : stream;
        const int rc = launch_forward(dp, d, L.valu_rows, L.mfma_tiles, L.n_tasks, static_cast<const uint16_t*>(q),
                                      static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), out, s);
        if (rc != 0)
            return set_error(KVATTN_EHIP, std::string("forward launch failed: ") + hipGetErrorString(hipError_t(rc)));
    }
    return KVATTN_OK;
}

kvattn_status run_merge(kvattn_plan_t plan, float* out, void* stream, void* ws = nullptr) {
    if (!out) return set_error(KVATTN_EINVAL, "out is NULL");
    if (plan->opts.new_token)
        return set_error(KVATTN_EINVAL, "the plan takes each query's newest token from the call: use kvattn_decode_append");
    const DevPlan dp = resolve(*plan, -1, ws ? ws : plan->dev_ws);
    const Dims d = dims(*plan);
    const int rc = launch_merge(dp, d, int(plan->merge_query.size()), out, stream);
    if (rc != 0) return set_error(KVATTN_EHIP, std::string("merge launch failed: ") + hipGetErrorString(hipError_t(rc)));
    return KVATTN_OK;
}

// Generation of the plan whose blob each device's static scratch holds (0: none).
std::mutex g_scratch_mu;
uint64_t g_scratch_generation[kMaxDevices] = {};

}  // namespace
}  // namespace kvattn

extern "C" {

kvattn_status kvattn_plan_upload(kvattn_plan_t plan, void* dev_workspace, size_t bytes, void* stream) {
    using namespace kvattn;
    clear_error();
    if (!plan || !dev_workspace) return set_error(KVATTN_EINVAL, "plan or dev_workspace is NULL");
    if ((reinterpret_cast<uintptr_t>(dev_workspace) & 255u) != 0)
        return set_error(KVATTN_EWORKSPACE, "dev_workspace must be 256-byte aligned");
    if (bytes < plan->header.total_bytes)
        return set_error(KVATTN_EWORKSPACE, "workspace holds " + std::to_string(bytes) + " bytes, plan needs " +
                                                std::to_string(plan->header.total_bytes));
    hipStream_t s = static_cast<hipStream_t>(stream);
    // A captured copy would read the host blob again at every replay, after
    // updates have changed it: uploads stay outside graphs.
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(s, &cap);
    if (e != hipSuccess) return set_error(KVATTN_EHIP, std::string("stream query failed: ") + hipGetErrorString(e));
    if (cap != hipStreamCaptureStatusNone)
        return set_error(KVATTN_EINVAL, "kvattn_plan_upload on a capturing stream: upload before capturing decodes");
    if (!plan->upload_event) {
        hipEvent_t ev = nullptr;
        e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
        if (e != hipSuccess) return set_error(KVATTN_EHIP, std::string("event creation failed: ") + hipGetErrorString(e));
        plan->upload_event = ev;
        plan->upload_wait = wait_upload_event;
    }
    // an earlier upload of this plan may still be reading the blob; it is
    // unchanged since (updates wait for it), so the copies may overlap
    e = hipMemcpyAsync(dev_workspace, plan->blob.data(), plan->blob.size(), hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return set_error(KVATTN_EHIP, std::string("upload copy failed: ") + hipGetErrorString(e));
    // kvattn_plan_update and kvattn_plan_destroy wait for this event before they
    // change or free the blob the copy reads
    e = hipEventRecord(static_cast<hipEvent_t>(plan->upload_event), s);
    if (e != hipSuccess) {
        (void)hipStreamSynchronize(s);   // no event to wait on later: let the copy finish now
        return set_error(KVATTN_EHIP, std::string("event record failed: ") + hipGetErrorString(e));
    }
    plan->dev_ws = dev_workspace;
    plan->dev_bytes = bytes;
    return KVATTN_OK;
}

kvattn_status kvattn_forward(const void* q, const void* k_cache, const void* v_cache, kvattn_plan_t plan, float* out,
                             void* stream) {
    using namespace kvattn;
    clear_error();
    kvattn_status s = check_bound(plan);
    if (s != KVATTN_OK) return s;
    return run_forward(q, k_cache, v_cache, plan, out, stream);
}

kvattn_status kvattn_merge(kvattn_plan_t plan, float* out, void* stream) {
    using namespace kvattn;
    clear_error();
    kvattn_status s = check_bound(plan);
    if (s != KVATTN_OK) return s;
    return run_merge(plan, out, stream);
}

kvattn_status kvattn_decode(const void* q, const void* k_cache, const void* v_cache, kvattn_plan_t plan, float* out,
                            void* stream) {
    using namespace kvattn;
    clear_error();
    kvattn_status s = check_bound(plan);
    if (s != KVATTN_OK) return s;
    if (plan->opts.new_token)
        return set_error(KVATTN_EINVAL, "the plan takes each query's newest token from the call: use kvattn_decode_append");
    s = run_forward(q, k_cache, v_cache, plan, out, stream);
    if (s != KVATTN_OK) return s;
    if (plan->fused_merge) return KVATTN_OK;   // the forward launch merged
    return run_merge(plan, out, stream);
}

kvattn_status kvattn_decode_append(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                   kvattn_plan_t plan, float* out, void* stream) {
    using namespace kvattn;
    clear_error();
    kvattn_status s = check_bound(plan);
    if (s != KVATTN_OK) return s;
    if (!plan->opts.new_token) return set_error(KVATTN_EINVAL, "the plan was made without new_token: use kvattn_decode");
    if (!k_new || !v_new) return set_error(KVATTN_EINVAL, "k_new or v_new is NULL");
    if (!aligned16(k_new) || !aligned16(v_new)) return set_error(KVATTN_EINVAL, "k_new and v_new must be 16-byte aligned");
    // the forward reads the cached parts only; the merge adds the new tokens and writes them into the cache
    s = run_forward(q, k_cache, v_cache, plan, out, stream);
    if (s != KVATTN_OK) return s;
    const DevPlan dp = resolve(*plan, -1, plan->dev_ws);
    const Dims d = dims(*plan);
    NewTokens nt;
    nt.q = static_cast<const uint16_t*>(q);
    nt.k_new = static_cast<const uint16_t*>(k_new);
    nt.v_new = static_cast<const uint16_t*>(v_new);
    nt.k_cache = static_cast<uint16_t*>(k_cache);
    nt.v_cache = static_cast<uint16_t*>(v_cache);
    const int rc = launch_merge_append(dp, d, int(plan->merge_query.size()), nt, out, stream);
    if (rc != 0) return set_error(KVATTN_EHIP, std::string("merge launch failed: ") + hipGetErrorString(hipError_t(rc)));
    return KVATTN_OK;
}

kvattn_status kvattn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, kvattn_plan_t plan,
                                    float* out, void* stream) {
    using namespace kvattn;
    clear_error();
    if (!plan) return set_error(KVATTN_EINVAL, "plan is NULL");
    if (plan->opts.new_token)
        return set_error(KVATTN_EINVAL, "the plan takes each query's newest token from the call: use kvattn_decode_append");
    if (plan->header.total_bytes > kNoallocScratchBytes)
        return set_error(KVATTN_EWORKSPACE, "the plan needs " + std::to_string(plan->header.total_bytes) +
                                                " bytes of workspace; the static scratch holds " +
                                                std::to_string(kNoallocScratchBytes) + ": use kvattn_decode");
    void* ws = nullptr;
    int rc = scratch_device_pointer(&ws);
    if (rc != 0) return set_error(KVATTN_EHIP, std::string("scratch lookup failed: ") + hipGetErrorString(hipError_t(rc)));
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return set_error(KVATTN_EHIP, std::string("device query failed: ") + hipGetErrorString(e));
    hipStream_t s = static_cast<hipStream_t>(stream);
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (g_scratch_generation[dev] != plan->generation) {
            // stage this plan's schedule (its claim counter zeroed) in the scratch
            hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
            e = hipStreamIsCapturing(s, &cap);
            if (e != hipSuccess) return set_error(KVATTN_EHIP, std::string("stream query failed: ") + hipGetErrorString(e));
            if (cap != hipStreamCaptureStatusNone)
                return set_error(KVATTN_EINVAL, "the plan is not staged in this device's scratch: call once before capturing");
            if (!plan->upload_event) {
                hipEvent_t ev = nullptr;
                e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
                if (e != hipSuccess) return set_error(KVATTN_EHIP, std::string("event creation failed: ") + hipGetErrorString(e));
                plan->upload_event = ev;
                plan->upload_wait = wait_upload_event;
            }
            e = hipMemcpyAsync(ws, plan->blob.data(), plan->blob.size(), hipMemcpyHostToDevice, s);
            if (e != hipSuccess) return set_error(KVATTN_EHIP, std::string("staging copy failed: ") + hipGetErrorString(e));
            e = hipEventRecord(static_cast<hipEvent_t>(plan->upload_event), s);
            if (e != hipSuccess) {
                (void)hipStreamSynchronize(s);
                return set_error(KVATTN_EHIP, std::string("event record failed: ") + hipGetErrorString(e));
            }
            g_scratch_generation[dev] = plan->generation;
        }
    }
    kvattn_status st = run_forward(q, k_cache, v_cache, plan, out, stream, nullptr, ws);
    if (st != KVATTN_OK) return st;
    if (plan->fused_merge) return KVATTN_OK;   // the forward launch merged
    return run_merge(plan, out, stream, ws);
}

kvattn_status kvattn_read_probe(const void* a, size_t a_bytes, const void* b, size_t b_bytes, void* sink,
                                size_t sink_bytes, int32_t grid, int32_t loads_in_flight, int32_t threads,
                                void* stream) {
    using namespace kvattn;
    clear_error();
    if (!a || !b || !sink) return set_error(KVATTN_EINVAL, "a, b or sink is NULL");
    if (!aligned16(a) || !aligned16(b) || !aligned16(sink) || (a_bytes & 15u) || (b_bytes & 15u))
        return set_error(KVATTN_EINVAL, "buffers must be 16-byte aligned and multiples of 16 bytes");
    if (grid < 1) return set_error(KVATTN_EINVAL, "grid must be >= 1");
    if ((loads_in_flight != 2 && loads_in_flight != 4 && loads_in_flight != 8) ||
        (threads != 256 && threads != 512 && threads != 1024))
        return set_error(KVATTN_EINVAL, "loads_in_flight must be 2, 4 or 8 and threads 256, 512 or 1024");
    if (sink_bytes < size_t(grid) * size_t(threads) * 4)
        return set_error(KVATTN_EINVAL, "sink holds " + std::to_string(sink_bytes) + " bytes, the probe writes " +
                                            std::to_string(size_t(grid) * size_t(threads) * 4));
    const int rc = launch_read_probe(a, a_bytes, b, b_bytes, static_cast<uint32_t*>(sink), grid, loads_in_flight,
                                     threads, stream);
    if (rc != 0) return set_error(KVATTN_EHIP, std::string("probe launch failed: ") + hipGetErrorString(hipError_t(rc)));
    return KVATTN_OK;
}

kvattn_status kvattn_decode_streams(const void* q, const void* k_cache, const void* v_cache, kvattn_plan_t plan,
                                    float* out, void* stream, void* side_stream) {
    using namespace kvattn;
    clear_error();
    kvattn_status s = check_bound(plan);
    if (s != KVATTN_OK) return s;
    if (!plan->opts.multi_stream)
        return set_error(KVATTN_EINVAL, "the plan was made without multi_stream: use kvattn_decode");
    if (plan->opts.new_token)
        return set_error(KVATTN_EINVAL, "the plan takes each query's newest token from the call: use kvattn_decode_append");
    if (side_stream == stream) return set_error(KVATTN_EINVAL, "side_stream must differ from stream");
    for (void** ev : {&plan->fork_event, &plan->join_event}) {
        if (*ev) continue;
        hipEvent_t e = nullptr;
        const hipError_t err = hipEventCreateWithFlags(&e, hipEventDisableTiming);
        if (err != hipSuccess) return set_error(KVATTN_EHIP, std::string("event creation failed: ") + hipGetErrorString(err));
        *ev = e;
    }
    hipStream_t main_s = static_cast<hipStream_t>(stream), side_s = static_cast<hipStream_t>(side_stream);
    hipEvent_t fork = static_cast<hipEvent_t>(plan->fork_event), join = static_cast<hipEvent_t>(plan->join_event);
    // the side stream starts after the work already on the main stream (the caller's inputs)
    hipError_t e = hipEventRecord(fork, main_s);
    if (e == hipSuccess) e = hipStreamWaitEvent(side_s, fork, 0);
    if (e != hipSuccess) return set_error(KVATTN_EHIP, std::string("stream fork failed: ") + hipGetErrorString(e));
    s = run_forward(q, k_cache, v_cache, plan, out, stream, side_stream);
    // join before any error return, so the side stream never runs past the call
    e = hipEventRecord(join, side_s);
    if (e == hipSuccess) e = hipStreamWaitEvent(main_s, join, 0);
    if (s != KVATTN_OK) return s;
    if (e != hipSuccess) return set_error(KVATTN_EHIP, std::string("stream join failed: ") + hipGetErrorString(e));
    return run_merge(plan, out, stream);
}

void kvattn_plan_destroy(kvattn_plan_t plan) {
    if (!plan) return;
    // an upload still in flight reads the blob freed below
    if (plan->upload_event) {
        (void)hipEventSynchronize(static_cast<hipEvent_t>(plan->upload_event));
        (void)hipEventDestroy(static_cast<hipEvent_t>(plan->upload_event));
    }
    // events exist only if kvattn_decode_streams ran, i.e. on a host with the HIP runtime
    if (plan->fork_event) (void)hipEventDestroy(static_cast<hipEvent_t>(plan->fork_event));
    if (plan->join_event) (void)hipEventDestroy(static_cast<hipEvent_t>(plan->join_event));
    delete plan;
}

}  // extern "C"
