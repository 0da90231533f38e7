// Two-level expert store: every expert block lives in pinned host memory;
// a pool of HBM slots holds the experts the routing used most recently
// ([Q] "The engine", items 2-3: an LRU cache of experts in front of the
// slow tier, GPU slots, and copies into the slots overlapped with compute;
// [D] "Making it faster": the same for the DeepSeek-shaped model).
//
// On this machine the slow tier is host memory behind PCIe and the kernels
// can read it directly: the per-layer pointer tables the decode kernels take
// hold, for every expert, either its pinned host block (read in place, no
// copy and no host synchronisation) or its HBM slot. The tier only moves
// blocks into slots and repoints table entries; the routing never has to
// reach the host before a layer runs.
//
// Ordering (every step is enqueued, nothing waits on the host):
//  1. the table entries of the previous update's newcomers are written on
//     the compute stream after that update's block copies (an event of the
//     copy stream), so a kernel sees a slot only once its block is there;
//  2. the victims' entries are repointed to their host blocks on the
//     compute stream, and an event recorded right after them completes when
//     every kernel that could still read a victim's slot has finished;
//  3. the copy stream waits for that event and then copies the newcomers'
//     blocks into the freed slots, overlapping the compute stream's work.
// All table writes a kernel can observe are therefore ordered on the
// compute stream with the kernels themselves; an entry always points at
// valid data.
#include "../../include/moe_fp4.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

namespace {

constexpr int kRing = 4;  // staging buffers for table values in flight

bool host_mapped(const void* p) {
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, p) != hipSuccess) return false;
    return at.type == hipMemoryTypeHost && at.devicePointer == p;
}

bool on_device(const void* p) {
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, p) != hipSuccess) return false;
    return at.type == hipMemoryTypeDevice;
}

}  // namespace

struct moe_tier {
    int E = 0, k = 0, layers = 0, n_slots = 0;
    size_t block_bytes = 0;
    uint8_t* host = nullptr;   // pinned blocks [layers][E]
    uint8_t* slots = nullptr;  // HBM slots [n_slots]
    void** table = nullptr;    // device [layers][E]
    std::vector<int32_t> slot_of;     // [layers*E]: slot, or -1 (host)
    std::vector<uint8_t> pending;     // slot assigned, table entry not yet written
    std::vector<int32_t> owner;       // [n_slots]: key or -1
    std::vector<uint64_t> last_use;   // [layers*E]: update step of the last use (0: never)
    uint64_t step = 0;
    moe_tier_stats st = {};
    hipStream_t copy = nullptr;
    hipEvent_t copied[kRing] = {};    // block copies of update r landed (copy stream)
    hipEvent_t drained = nullptr;     // compute stream past the victims' repointing
    hipEvent_t staged[kRing] = {};    // table writes of ring entry r done (compute stream)
    void** stage = nullptr;           // pinned [kRing][2 * n_slots + 1] table values
    std::vector<int32_t> newcomers[kRing];
    int ring = 0;
    bool copied_valid[kRing] = {};

    void* host_block(int key) const { return host + (size_t)key * block_bytes; }
    void* slot_ptr(int s) const { return slots + (size_t)s * block_bytes; }
};

extern "C" {

int moe_tier_create(const moe_desc* d, int32_t layers, void* host_blocks, void* slots, int32_t n_slots,
                    void** table, moe_tier** out) {
    if (!out) return MOE_ERR_ARG;
    *out = nullptr;
    const size_t bb = moe_block_bytes(d);
    if (!bb) return MOE_ERR_ARG;
    if (layers < 1 || n_slots < 0 || !host_blocks || !table || (n_slots > 0 && !slots)) return MOE_ERR_ARG;
    if ((size_t)layers * d->E > (size_t)1 << 24) return MOE_ERR_ARG;
    if (bb % 256 || reinterpret_cast<uintptr_t>(host_blocks) % 256 || reinterpret_cast<uintptr_t>(slots) % 256 ||
        reinterpret_cast<uintptr_t>(table) % 8)
        return MOE_ERR_ARG;
    const size_t total = (size_t)layers * d->E * bb;
    // both ends of the host range must be pinned and mapped at the same
    // address (the kernels read misses in place); slots and table on the GPU
    if (!host_mapped(host_blocks) || !host_mapped(static_cast<uint8_t*>(host_blocks) + total - 1)) return MOE_ERR_ARG;
    if (!on_device(table) || (n_slots > 0 && (!on_device(slots) ||
                                              !on_device(static_cast<uint8_t*>(slots) + (size_t)n_slots * bb - 1))))
        return MOE_ERR_ARG;

    moe_tier* t = new (std::nothrow) moe_tier();
    if (!t) return MOE_ERR_ARG;
    t->E = d->E;
    t->k = d->k;
    t->layers = layers;
    t->n_slots = n_slots;
    t->block_bytes = bb;
    t->host = static_cast<uint8_t*>(host_blocks);
    t->slots = static_cast<uint8_t*>(slots);
    t->table = table;
    const size_t nkeys = (size_t)layers * d->E;
    t->slot_of.assign(nkeys, -1);
    t->pending.assign(nkeys, 0);
    t->owner.assign(n_slots, -1);
    t->last_use.assign(nkeys, 0);
    bool ok = hipStreamCreateWithFlags(&t->copy, hipStreamNonBlocking) == hipSuccess &&
              hipEventCreateWithFlags(&t->drained, hipEventDisableTiming) == hipSuccess;
    for (int r = 0; r < kRing && ok; r++)
        ok = hipEventCreateWithFlags(&t->copied[r], hipEventDisableTiming) == hipSuccess &&
             hipEventCreateWithFlags(&t->staged[r], hipEventDisableTiming) == hipSuccess;
    const size_t stage_n = std::max(nkeys, (size_t)kRing * (2 * n_slots + 1));
    ok = ok && hipHostMalloc(reinterpret_cast<void**>(&t->stage), stage_n * sizeof(void*), hipHostMallocDefault) ==
                   hipSuccess;
    if (ok) {
        // every entry starts at its host block
        for (size_t i = 0; i < nkeys; i++) t->stage[i] = t->host_block((int)i);
        ok = hipMemcpyAsync(table, t->stage, nkeys * sizeof(void*), hipMemcpyHostToDevice, t->copy) == hipSuccess &&
             hipStreamSynchronize(t->copy) == hipSuccess;
    }
    if (!ok) {
        moe_tier_destroy(t);
        return MOE_ERR_HIP;
    }
    *out = t;
    return MOE_OK;
}

int moe_tier_destroy(moe_tier* t) {
    if (!t) return MOE_OK;
    int rc = MOE_OK;
    auto chk = [&rc](hipError_t e) {
        if (e != hipSuccess) rc = MOE_ERR_HIP;
    };
    if (t->copy) chk(hipStreamSynchronize(t->copy));
    for (int r = 0; r < kRing; r++)
        if (t->staged[r]) chk(hipEventSynchronize(t->staged[r]));
    for (int r = 0; r < kRing; r++) {
        if (t->copied[r]) chk(hipEventDestroy(t->copied[r]));
        if (t->staged[r]) chk(hipEventDestroy(t->staged[r]));
    }
    if (t->drained) chk(hipEventDestroy(t->drained));
    if (t->copy) chk(hipStreamDestroy(t->copy));
    if (t->stage) chk(hipHostFree(t->stage));
    delete t;
    return rc;
}

int moe_tier_update(moe_tier* t, const int32_t* idx_host, int32_t max_promote, void* compute_stream) {
    if (!t || !idx_host || max_promote < 0) return MOE_ERR_ARG;
    hipStream_t cs = static_cast<hipStream_t>(compute_stream);
    const int r = t->ring;
    t->ring = (t->ring + 1) % kRing;
    // the staging entry r is rewritten below: its previous table writes must
    // have been performed (a host wait on an event kRing updates old)
    if (hipEventSynchronize(t->staged[r]) != hipSuccess) return MOE_ERR_HIP;
    void** stg = t->stage + (size_t)r * (2 * t->n_slots + 1);
    int nst = 0;

    // 1. newcomers of the previous update: their blocks are in (event), so
    // their entries switch to the slots, in order with the compute stream
    const int pr = (r + kRing - 1) % kRing;
    if (t->copied_valid[pr] && !t->newcomers[pr].empty()) {
        if (hipStreamWaitEvent(cs, t->copied[pr], 0) != hipSuccess) return MOE_ERR_HIP;
        for (int key : t->newcomers[pr]) {
            stg[nst] = t->slot_ptr(t->slot_of[key]);
            if (hipMemcpyAsync(t->table + key, stg + nst, sizeof(void*), hipMemcpyHostToDevice, cs) != hipSuccess)
                return MOE_ERR_HIP;
            nst++;
            t->pending[key] = 0;
        }
        t->newcomers[pr].clear();
    }
    t->copied_valid[pr] = false;

    // 2. the routing of this step: hits, misses, candidates in order
    t->step++;
    std::vector<int32_t> cand;
    for (int l = 0; l < t->layers; l++)
        for (int j = 0; j < t->k; j++) {
            const int e = idx_host[(size_t)l * t->k + j];
            if ((unsigned)e >= (unsigned)t->E) continue;
            const int key = l * t->E + e;
            const bool resident = t->slot_of[key] >= 0 && !t->pending[key];
            if (resident)
                t->st.hits++;
            else
                t->st.misses++;
            if (t->last_use[key] != t->step && t->slot_of[key] < 0) cand.push_back(key);
            t->last_use[key] = t->step;
        }

    // 3. victims: free slots first, then the least recently used resident
    // expert that this step did not use; pending slots are never victims
    std::vector<int32_t>& nc = t->newcomers[r];
    nc.clear();
    for (int key : cand) {
        if ((int)nc.size() >= max_promote) break;
        int best = -1;
        uint64_t best_use = UINT64_MAX;
        for (int s = 0; s < t->n_slots; s++) {
            const int o = t->owner[s];
            if (o < 0) {
                best = s;
                break;
            }
            if (t->pending[o] || t->last_use[o] == t->step) continue;
            if (t->last_use[o] < best_use) {
                best_use = t->last_use[o];
                best = s;
            }
        }
        if (best < 0) break;  // every slot holds an expert of this step
        const int v = t->owner[best];
        if (v >= 0) {
            stg[nst] = t->host_block(v);
            if (hipMemcpyAsync(t->table + v, stg + nst, sizeof(void*), hipMemcpyHostToDevice, cs) != hipSuccess)
                return MOE_ERR_HIP;
            nst++;
            t->slot_of[v] = -1;
            t->st.evictions++;
        }
        t->owner[best] = key;
        t->slot_of[key] = best;
        t->pending[key] = 1;
        nc.push_back(key);
    }
    if (hipEventRecord(t->staged[r], cs) != hipSuccess) return MOE_ERR_HIP;

    // 4. block copies on the copy stream once the compute stream is past the
    // victims' repointing (every kernel that could read a victim's slot is
    // done by then)
    if (!nc.empty()) {
        if (hipEventRecord(t->drained, cs) != hipSuccess || hipStreamWaitEvent(t->copy, t->drained, 0) != hipSuccess)
            return MOE_ERR_HIP;
        for (int key : nc)
            if (hipMemcpyAsync(t->slot_ptr(t->slot_of[key]), t->host_block(key), t->block_bytes,
                               hipMemcpyHostToDevice, t->copy) != hipSuccess)
                return MOE_ERR_HIP;
        if (hipEventRecord(t->copied[r], t->copy) != hipSuccess) return MOE_ERR_HIP;
        t->copied_valid[r] = true;
        t->st.promotions += (int64_t)nc.size();
    }
    return MOE_OK;
}

int moe_tier_get_stats(const moe_tier* t, moe_tier_stats* out) {
    if (!t || !out) return MOE_ERR_ARG;
    *out = t->st;
    int64_t res = 0, pend = 0;
    for (size_t i = 0; i < t->slot_of.size(); i++) {
        if (t->slot_of[i] >= 0 && !t->pending[i]) res++;
        if (t->pending[i]) pend++;
    }
    out->resident = res;
    out->pending = pend;
    return MOE_OK;
}

int32_t moe_tier_slot_of(const moe_tier* t, int32_t layer, int32_t expert) {
    if (!t || layer < 0 || layer >= t->layers || expert < 0 || expert >= t->E) return -1;
    const int key = layer * t->E + expert;
    return t->pending[key] ? -1 : t->slot_of[key];
}

}  // extern "C"
