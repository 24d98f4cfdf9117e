// C ABI of the decode library: argument checks, workspace cache, launches.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "../../include/mqa_decode.h"
#include "kernel_common.hpp"
#include "launch.hpp"
#include "plan.hpp"

namespace {

using mqa::Plan;

// Split-K scratch per (device, stream), grown on demand: one buffer for the
// partial outputs and LSEs, and a separate one for the fused combine's
// counters.  The counters are zeroed when allocated and every call leaves them
// at zero, so nothing else may ever write that buffer.
struct Workspace {
    void* ptr = nullptr;
    size_t bytes = 0;
    uint32_t* counters = nullptr;
    size_t ncounters = 0;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, uintptr_t>, Workspace> g_ws;

// Scratch of the no-allocation entry point (mqa_decode_attention_noalloc):
// the split partials live in this file-scope device array instead of a
// hipMalloc'd workspace.  Each device holds its own copy at its own address.
// In host code `scratch` names a host-side stand-in, never the device memory:
// the device address comes from hipGetSymbolAddress (scratch_address), and
// only that address is handed to kernels.
constexpr size_t kScratchBytes = (size_t)MQA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

mqa_status hip_fail(hipError_t e, const char* what) {
    mqa::set_error(std::string(what) + ": " + hipGetErrorString(e));
    return MQA_ERR_HIP;
}

mqa_status get_workspace(hipStream_t stream, size_t bytes, size_t ncounters, void** out,
                         uint32_t** counters_out) {
    *out = nullptr;
    *counters_out = nullptr;
    if (bytes == 0 && ncounters == 0) return MQA_OK;
    // Fault injection for tests: MQA_FAIL_WORKSPACE_ALLOC=1 makes every
    // workspace allocation fail, before any HIP call.
    if (const char* f = std::getenv("MQA_FAIL_WORKSPACE_ALLOC")) {
        if (f[0] == '1') {
            mqa::set_error("split-K workspace allocation failed (MQA_FAIL_WORKSPACE_ALLOC is set)");
            return MQA_ERR_WORKSPACE;
        }
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace& ws = g_ws[{dev, reinterpret_cast<uintptr_t>(stream)}];
    const bool grow_parts = ws.bytes < bytes;
    const bool grow_counters = ws.ncounters < ncounters;
    if ((grow_parts && ws.ptr) || (grow_counters && ws.counters)) {
        // The old buffers may still be in use by work queued on this stream.
        e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    }
    if (grow_parts) {
        if (ws.ptr) {
            e = hipFree(ws.ptr);
            ws.ptr = nullptr;
            ws.bytes = 0;
            if (e != hipSuccess) return hip_fail(e, "hipFree");
        }
        void* p = nullptr;
        e = hipMalloc(&p, bytes);
        if (e != hipSuccess) {
            mqa::set_error(std::string("hipMalloc of split-K workspace failed: ") + hipGetErrorString(e));
            return MQA_ERR_WORKSPACE;
        }
        ws.ptr = p;
        ws.bytes = bytes;
    }
    if (grow_counters) {
        if (ws.counters) {
            e = hipFree(ws.counters);
            ws.counters = nullptr;
            ws.ncounters = 0;
            if (e != hipSuccess) return hip_fail(e, "hipFree");
        }
        void* p = nullptr;
        e = hipMalloc(&p, ncounters * sizeof(uint32_t));
        if (e != hipSuccess) {
            mqa::set_error(std::string("hipMalloc of arrival counters failed: ") + hipGetErrorString(e));
            return MQA_ERR_WORKSPACE;
        }
        e = hipMemset(p, 0, ncounters * sizeof(uint32_t));
        if (e != hipSuccess) {
            (void)hipFree(p);
            return hip_fail(e, "hipMemset of arrival counters");
        }
        ws.counters = static_cast<uint32_t*>(p);
        ws.ncounters = ncounters;
    }
    *out = ws.ptr;
    *counters_out = ws.counters;
    return MQA_OK;
}

// Device address of this device's `scratch`, looked up once per device with
// that device current (the first no-allocation call on it).
mqa_status scratch_address(void** out) {
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) {
        mqa::set_error("device index beyond the scratch table");
        return MQA_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) {
            mqa::set_error("hipGetSymbolAddress(scratch) returned NULL");
            return MQA_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MQA_OK;
}

// Checks the no-allocation entry point adds to the plan: the separate combine
// only (nothing in the scratch then has to start at zero) and a workspace that
// fits the scratch.  Host only, before any HIP call.
mqa_status check_noalloc(const Plan& plan) {
    if (plan.combine == 2) {
        mqa::set_error("the no-allocation entry point merges split sequences with the separate combine kernel "
                       "only (combine = 2 is not available)");
        return MQA_ERR_ARG;
    }
    if (plan.workspace_bytes > kScratchBytes) {
        mqa::set_error("this call needs " + std::to_string(plan.workspace_bytes) +
                       " bytes of split scratch; the no-allocation entry point holds " +
                       std::to_string(kScratchBytes) + " (use mqa_decode_attention_ex, or larger chunks)");
        return MQA_ERR_WORKSPACE;
    }
    return MQA_OK;
}

mqa_status run(const void* q, const void* k, const void* v, const int32_t* seq_lens, float* out,
               int B, int Hq, int Hkv, int D, int Lmax, float scale, void* stream_ptr,
               const mqa_decode_opts* opts, const mqa::PagedCache* paged = nullptr, int T = 1,
               bool noalloc = false) {
    mqa::set_error("");
    Plan plan;
    mqa_status st = mqa::make_plan(B, Hq, Hkv, D, Lmax, scale, opts, 0, &plan, T);
    if (st != MQA_OK) return st;
    st = mqa::check_pointers(B, Lmax, q, k, v, seq_lens, out);
    if (st != MQA_OK) return st;
    const float* k_scale = opts ? opts->k_scale : nullptr;
    const float* v_scale = opts ? opts->v_scale : nullptr;
    if (plan.kv_format != MQA_KV_BF16 && B > 0 && Lmax > 0) {
        if (!k_scale || !v_scale) {
            mqa::set_error("k_scale and v_scale must be non-NULL for an 8-bit cache");
            return MQA_ERR_NULL;
        }
        if (((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) & 3u) != 0) {
            mqa::set_error("k_scale and v_scale must be 4-byte aligned");
            return MQA_ERR_ALIGN;
        }
    }
    if (noalloc) {
        st = check_noalloc(plan);
        if (st != MQA_OK) return st;
        // the persistent schedule's queue needs memory that starts at zero
        if (opts && opts->schedule == 2) {
            mqa::set_error("the no-allocation entry point runs one workgroup per work item (schedule 2 is not "
                           "available)");
            return MQA_ERR_ARG;
        }
        if (plan.persist) {
            plan.persist = 0;
            plan.counters -= mqa::kPersistCounters;
        }
    }
    if (B == 0) return MQA_OK;

    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
    void* ws = nullptr;
    uint32_t* counters = nullptr;
    if (noalloc) {
        if (plan.workspace_bytes > 0) {
            st = scratch_address(&ws);
            if (st != MQA_OK) return st;
        }
    } else {
        st = get_workspace(stream, plan.workspace_bytes, plan.counters, &ws, &counters);
        if (st != MQA_OK) return st;
    }

    mqa::DecodeArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = k;
    a.v = v;
    if (plan.kv_format != MQA_KV_BF16) {
        a.k_scale = k_scale;
        a.v_scale = v_scale;
    }
    a.seq_lens = seq_lens;
    a.out = out;
    a.part_o = ws ? reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + plan.part_o_offset) : nullptr;
    a.part_ml = ws ? reinterpret_cast<mqa::f32x2_t*>(static_cast<char*>(ws) + plan.part_ml_offset) : nullptr;
    a.counters = counters;
    if (plan.persist) {
        a.queue = counters + (plan.counters - mqa::kPersistCounters);
        a.items = plan.grid_main * plan.head_blocks;
        a.grid_x = plan.grid_main;
    }
    if (paged) {
        a.block_table = paged->block_table;
        a.page_shift = paged->page_shift;
        a.max_blocks = paged->max_blocks;
        a.num_pages = paged->num_pages;
    }
    a.units = plan.rows * Hkv;
    a.fused = plan.combine == 2 ? 1 : 0;
    a.fused_wait = mqa::kFusedWaitTicks;
    if (a.fused) {
        if (const char* t = std::getenv("MQA_FUSED_WAIT_TICKS")) {
            // at most 10 ms: a workgroup whose partners cannot become resident
            // holds its CU for this long before it leaves its part to them
            const unsigned long v = std::strtoul(t, nullptr, 10);
            a.fused_wait = (uint32_t)(v < mqa::kFusedMaxWaitTicks ? v : mqa::kFusedMaxWaitTicks);
        }
    }
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.D = D;
    a.Lmax = Lmax;
    a.G = plan.G;
    a.T = plan.T;
    a.GT = plan.GT;
    a.chunk = plan.chunk;
    a.max_splits = plan.max_splits;
    a.window = plan.window;
    a.qk_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)

    hipEvent_t ev0 = opts ? static_cast<hipEvent_t>(opts->ev_main_begin) : nullptr;
    hipEvent_t ev1 = opts ? static_cast<hipEvent_t>(opts->ev_main_end) : nullptr;
    hipError_t e;
    if (plan.variant == MQA_VARIANT_VALU)
        e = mqa::launch_decode_valu(plan, a, stream, ev0, ev1);
    else
        e = mqa::launch_decode_mfma(plan, a, stream, ev0, ev1);
    if (e != hipSuccess) return hip_fail(e, "split-K kernel launch");
    if (plan.combine == 1) {
        mqa::CombineArgs c{};
        c.part_o = a.part_o;
        c.part_ml = a.part_ml;
        c.seq_lens = seq_lens;
        c.out = out;
        c.Hq = Hq;
        c.Hkv = Hkv;
        c.D = D;
        c.Lmax = Lmax;
        c.G = plan.G;
        c.T = plan.T;
        c.GT = plan.GT;
        c.chunk = plan.chunk;
        c.max_splits = plan.max_splits;
        c.window = a.window;
        c.dsplit = plan.combine_dsplit;
        e = mqa::launch_combine(plan, c, stream, opts ? static_cast<hipEvent_t>(opts->ev_combine_begin) : nullptr,
                                opts ? static_cast<hipEvent_t>(opts->ev_combine_end) : nullptr);
        if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
    }
    return MQA_OK;
}

}  // namespace

extern "C" {

mqa_status mqa_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* seq_lens, float* out, int B, int Hq, int Hkv,
                                int D, int Lmax, float scale, void* stream) {
    return run(q, k_cache, v_cache, seq_lens, out, B, Hq, Hkv, D, Lmax, scale, stream, nullptr);
}

mqa_status mqa_decode_attention_ex(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* seq_lens, float* out, int B, int Hq, int Hkv,
                                   int D, int Lmax, float scale, void* stream,
                                   const mqa_decode_opts* opts) {
    return run(q, k_cache, v_cache, seq_lens, out, B, Hq, Hkv, D, Lmax, scale, stream, opts);
}

mqa_status mqa_decode_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* seq_lens, float* out, int B, int Hq, int Hkv,
                                        int D, int Lmax, float scale, void* stream,
                                        const mqa_decode_opts* opts) {
    return run(q, k_cache, v_cache, seq_lens, out, B, Hq, Hkv, D, Lmax, scale, stream, opts, nullptr, 1,
               true);
}

mqa_status mqa_decode_attention_window(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* seq_lens, float* out, int B, int Hq, int Hkv,
                                       int D, int Lmax, int window, float scale, void* stream) {
    if (window < 1) {
        mqa::set_error("window must be >= 1");
        return MQA_ERR_ARG;
    }
    mqa_decode_opts o{};
    o.window = window;
    return run(q, k_cache, v_cache, seq_lens, out, B, Hq, Hkv, D, Lmax, scale, stream, &o);
}

mqa_status mqa_decode_attention_quant(const void* q, const void* k_codes, const void* v_codes,
                                      const float* k_scale, const float* v_scale, const int32_t* seq_lens,
                                      float* out, int B, int Hq, int Hkv, int D, int Lmax, int kv_format,
                                      float scale, void* stream, const mqa_decode_opts* opts) {
    if (kv_format != MQA_KV_FP8_E4M3 && kv_format != MQA_KV_INT8) {
        mqa::set_error("kv_format must be MQA_KV_FP8_E4M3 or MQA_KV_INT8");
        return MQA_ERR_ARG;
    }
    mqa_decode_opts o{};
    if (opts) o = *opts;
    o.kv_format = kv_format;
    o.k_scale = k_scale;
    o.v_scale = v_scale;
    return run(q, k_codes, v_codes, seq_lens, out, B, Hq, Hkv, D, Lmax, scale, stream, &o);
}

mqa_status mqa_decode_attention_multi(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* seq_lens, float* out, int B, int T, int Hq, int Hkv,
                                      int D, int Lmax, float scale, void* stream, const mqa_decode_opts* opts) {
    return run(q, k_cache, v_cache, seq_lens, out, B, Hq, Hkv, D, Lmax, scale, stream, opts, nullptr, T);
}

mqa_status mqa_decode_attention_paged(const void* q, const void* k_pages, const void* v_pages,
                                      const int32_t* block_table, const int32_t* seq_lens, float* out,
                                      int B, int Hq, int Hkv, int D, int num_pages, int page_size,
                                      int max_blocks, float scale, void* stream,
                                      const mqa_decode_opts* opts) {
    mqa::set_error("");
    mqa::PagedCache pc{};
    int Lmax = 0;
    const mqa_status st = mqa::check_paged(B, block_table, num_pages, page_size, max_blocks, &pc, &Lmax);
    if (st != MQA_OK) return st;
    return run(q, k_pages, v_pages, seq_lens, out, B, Hq, Hkv, D, Lmax, scale, stream, opts, &pc);
}

mqa_status mqa_prefill_attention(const void* q_seq, const void* k_cache, const void* v_cache,
                                 const int32_t* seq_lens, float* out_seq, int B, int Hq, int Hkv,
                                 int D, int Lmax, float scale, void* stream) {
    mqa::set_error("");
    Plan plan;
    mqa_status st = mqa::make_plan(B, Hq, Hkv, D, Lmax, scale, nullptr, mqa::kCausalPrefill, &plan);
    if (st != MQA_OK) return st;
    st = mqa::check_pointers(B, Lmax, q_seq, k_cache, v_cache, seq_lens, out_seq);
    if (st != MQA_OK) return st;
    if (plan.grid_main == 0) return MQA_OK;
    mqa::PrefillArgs a{};
    a.q = static_cast<const uint16_t*>(q_seq);
    a.k = static_cast<const uint16_t*>(k_cache);
    a.v = static_cast<const uint16_t*>(v_cache);
    a.seq_lens = seq_lens;
    a.out = out_seq;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.D = D;
    a.Lmax = Lmax;
    a.G = plan.G;
    a.row_blocks = plan.row_blocks;
    a.qk_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)
    const hipError_t e = mqa::launch_prefill_mfma(plan, a, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "prefill kernel launch");
    return MQA_OK;
}

mqa_status mqa_prefill_plan(int B, int Hq, int Hkv, int D, int Lmax, float scale, mqa_plan_info* info,
                            int* rows_per_block) {
    mqa::set_error("");
    Plan p;
    const mqa_status st = mqa::make_plan(B, Hq, Hkv, D, Lmax, scale, nullptr, mqa::kCausalPrefill, &p);
    if (st != MQA_OK) return st;
    if (info) {
        info->variant = p.variant;
        info->chunk = p.chunk;
        info->max_splits = p.max_splits;
        info->combine = p.combine;
        info->head_blocks = p.head_blocks;
        info->grid_main = p.grid_main * p.head_blocks;
        info->block_main = p.block_main;
        info->grid_combine = p.grid_combine;
        info->workspace_bytes = p.workspace_bytes;
        info->persistent = p.persist;
    }
    if (rows_per_block) *rows_per_block = p.heads_per_block;
    return MQA_OK;
}

mqa_status mqa_decode_plan(int B, int Hq, int Hkv, int D, int Lmax, float scale,
                           const mqa_decode_opts* opts, mqa_plan_info* info) {
    return mqa_decode_plan_multi(B, 1, Hq, Hkv, D, Lmax, scale, opts, info);
}

mqa_status mqa_decode_plan_multi(int B, int T, int Hq, int Hkv, int D, int Lmax, float scale,
                                 const mqa_decode_opts* opts, mqa_plan_info* info) {
    mqa::set_error("");
    Plan p;
    const mqa_status st = mqa::make_plan(B, Hq, Hkv, D, Lmax, scale, opts, 0, &p, T);
    if (st != MQA_OK) return st;
    if (info) {
        info->variant = p.variant;
        info->chunk = p.chunk;
        info->max_splits = p.max_splits;
        info->combine = p.combine;
        info->head_blocks = p.head_blocks;
        info->grid_main = p.grid_main * p.head_blocks;
        info->block_main = p.block_main;
        info->grid_combine = p.grid_combine;
        info->workspace_bytes = p.workspace_bytes;
        info->persistent = p.persist;
    }
    return MQA_OK;
}

const char* mqa_status_string(mqa_status s) {
    // A C caller may pass any int; read it as one, since a C++ load of an
    // enum outside its enumerators' range is undefined.
    int v;
    std::memcpy(&v, &s, sizeof v);
    switch (v) {
        case MQA_OK: return "ok";
        case MQA_ERR_NULL: return "null pointer argument";
        case MQA_ERR_SHAPE: return "invalid shape";
        case MQA_ERR_UNSUPPORTED: return "unsupported shape";
        case MQA_ERR_ALIGN: return "misaligned pointer";
        case MQA_ERR_WORKSPACE: return "workspace allocation failed";
        case MQA_ERR_HIP: return "HIP runtime error";
        case MQA_ERR_ARG: return "invalid argument";
    }
    return "unknown status";
}

const char* mqa_last_error(void) { return mqa::last_error(); }

void mqa_release_workspaces(void) {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    for (auto& kv : g_ws) {
        if (kv.second.ptr || kv.second.counters) {
            int prev = 0;
            (void)hipGetDevice(&prev);
            (void)hipSetDevice(kv.first.first);
            if (kv.second.ptr) (void)hipFree(kv.second.ptr);
            if (kv.second.counters) (void)hipFree(kv.second.counters);
            (void)hipSetDevice(prev);
        }
    }
    g_ws.clear();
}

mqa_status mqa_stream_read_probe(const void* buf, size_t bytes, int workgroups, uint32_t* sink, void* stream,
                                 void* ev_begin, void* ev_end) {
    mqa::set_error("");
    if (bytes == 0) return MQA_OK;
    if (!buf || !sink) {
        mqa::set_error("buf and sink must be non-NULL");
        return MQA_ERR_NULL;
    }
    if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || (bytes & 15u) != 0 ||
        (reinterpret_cast<uintptr_t>(sink) & 3u) != 0) {
        mqa::set_error("buf must be 16-byte aligned, bytes a multiple of 16 and sink 4-byte aligned");
        return MQA_ERR_ALIGN;
    }
    if (workgroups < 1 || workgroups > (1 << 24)) {
        mqa::set_error("workgroups must be in [1, 2^24]");
        return MQA_ERR_ARG;
    }
    if ((bytes + (size_t)workgroups - 1) / (size_t)workgroups > ((size_t)1 << 30)) {
        mqa::set_error("each workgroup's slice must be at most 1 GiB");
        return MQA_ERR_UNSUPPORTED;
    }
    const hipError_t e = mqa::launch_stream_read(buf, (long long)bytes, workgroups, sink,
                                                 reinterpret_cast<hipStream_t>(stream),
                                                 static_cast<hipEvent_t>(ev_begin), static_cast<hipEvent_t>(ev_end));
    if (e != hipSuccess) return hip_fail(e, "stream-read kernel launch");
    return MQA_OK;
}

int mqa_version(void) { return 10600; }  // 1.6.0

}  // extern "C"
