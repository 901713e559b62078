// spec_verify_api.hip -- the C ABI declared in include/spec_verify.h.
//
// Host side only: argument checks, workspace layout, kernel launches on the
// caller's stream.  Nothing here allocates device memory or synchronises.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "../../include/spec_verify.h"
#include "sv_common.h"
#include "sv_launch.h"

// Scratch of spec_verify_step_noalloc, for callers that cannot allocate:
// one copy per GPU in the library's code object, held until the process
// ends.  Host code never passes the array's name to a kernel (on the host it
// is a stand-in, not a device address): the address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

thread_local const char* g_detail = "";

constexpr int kMaxK = 63;                          // K+1 positions scanned by one wave64
constexpr int kMaxV = 1024 * sv::kChunk;           // the residual prefix lives in LDS
constexpr int kMaxDevices = 64;

std::atomic<int> g_cus[kMaxDevices];
std::atomic<void*> g_scratch[kMaxDevices];   // device address of `scratch`, per device
// rounds a workgroup of the one-launch accept + residual polls for its
// sequence's chunk sums before it sums every chunk itself
std::atomic<int> g_poll_limit{sv::kDefaultPollLimit};
int poll_limit() { return g_poll_limit.load(std::memory_order_relaxed); }
// poll slots per sequence the accept kernel zeroes for the residual draw of
// n sequences that follows (one per chunk when that draw polls, else none)
int residual_slots(int n, int V) { return sv::residual_poll_group(n, V) > 0 ? sv::n_chunks(V) : 0; }

spec_status_t hip_fail(hipError_t e) {
    g_detail = hipGetErrorString(e);
    return SPEC_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// B >= 1, 0 <= K <= 63, 1 <= V <= kMaxV, and every grid the calls launch fits
// in 31 bits.
bool sizes_ok(int B, int K, int V) {
    if (B < 1 || K < 0 || K > kMaxK || V < 1 || V > kMaxV) return false;
    const long long jobs = (long long)B * (2 * K + 1);
    return jobs * sv::n_chunks(V) <= 0x7fffffffLL && (long long)B * (K + 1) <= 0x7fffffffLL;
}

hipError_t num_cus(int* out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) {
        const int cached = g_cus[dev].load(std::memory_order_relaxed);
        if (cached > 0) {
            *out = cached;
            return hipSuccess;
        }
    }
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (n < 1) n = 1;
    if (dev >= 0 && dev < kMaxDevices) g_cus[dev].store(n, std::memory_order_relaxed);
    *out = n;
    return hipSuccess;
}

// The current device's copy of `scratch`: looked up on the first call made
// with that device current, then cached (two threads racing on the first
// call store the same address).
hipError_t scratch_ptr(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Workspace {
    sv::StatRec* stats;
    sv::AcceptInfo* info;
    float* sums;
    int* counters;
    unsigned long long* slots;   // poll slots of the one-launch accept + residual, right after the counters' block
};

// Layout for up to B selected rows: chunk statistics of B*(K+1) target rows and
// B*K draft rows, one AcceptInfo per row, the residual chunk sums, and one
// completion counter per row followed by the poll slots of the one-launch
// accept + residual (both zeroed by the kernel that runs before it).
size_t workspace_layout(int B, int K, int V, void* base, Workspace* ws) {
    const size_t nc = (size_t)sv::n_chunks(V);
    const size_t stats = align256(((size_t)B * (K + 1) + (size_t)B * K) * nc * sizeof(sv::StatRec));
    const size_t info = align256((size_t)B * sizeof(sv::AcceptInfo));
    // residual chunk sums: one per statistics chunk, or per (smaller) chunk of
    // the one-launch accept + residual, whichever is more
    const size_t sums = align256((size_t)B * std::max(nc, (size_t)sv::n_fused_chunks(V)) * sizeof(float));
    const size_t counter_block = align256((size_t)B * sizeof(int));
    const size_t counters = counter_block + align256((size_t)sv::kPollMaxSlots * sizeof(unsigned long long));
    if (ws) {
        char* p = static_cast<char*>(base);
        ws->stats = reinterpret_cast<sv::StatRec*>(p);
        ws->info = reinterpret_cast<sv::AcceptInfo*>(p + stats);
        ws->sums = reinterpret_cast<float*>(p + stats + info);
        ws->counters = reinterpret_cast<int*>(p + stats + info + sums);
        ws->slots = reinterpret_cast<unsigned long long*>(p + stats + info + sums + counter_block);
    }
    return stats + info + sums + counters;
}

spec_status_t check_accept_common(const float* logits, const int32_t* draft_tokens, const int32_t* rows,
                                  int n_rows, int B, int K, int V, bool has_drafts, const int32_t* accepted_len,
                                  const int32_t* out_tokens, void* workspace, size_t workspace_bytes) {
    if (!sizes_ok(B, K, V)) return SPEC_ERR_ARG;
    if (!logits || !accepted_len || !out_tokens) return SPEC_ERR_ARG;
    if (has_drafts && !draft_tokens) return SPEC_ERR_ARG;
    if (rows && (n_rows < 0 || n_rows > B)) return SPEC_ERR_ARG;
    if (!aligned16(logits)) return SPEC_ERR_ALIGN;
    if (!workspace || workspace_bytes < workspace_layout(B, K, V, nullptr, nullptr)) return SPEC_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SPEC_ERR_ALIGN;
    return SPEC_OK;
}

// ragged batches: row_start[B+1] on the device, total target rows declared by
// the caller (B <= total <= B*(K_max+1))
spec_status_t check_ragged(const int32_t* row_start, int total_rows, int B, int K) {
    if (!row_start) return SPEC_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(row_start) & 3u) != 0) return SPEC_ERR_ALIGN;
    if (B < 1 || total_rows < B || (long long)total_rows > (long long)B * (K + 1)) return SPEC_ERR_ARG;
    return SPEC_OK;
}

// records written by the statistics pass: target slots, then draft slots
sv::RecLayout pass_layout(const sv::StatRec* stats, int n_rows, int K, int V) {
    const int nc = sv::n_chunks(V);
    return sv::RecLayout{stats, nc, false, stats + (size_t)n_rows * (K + 1) * nc, nc, false};
}

spec_status_t greedy_impl(const float* logits, const int32_t* draft_tokens, const int32_t* rows, int n_rows,
                          sv::SeqRows seq, int V, int32_t* accepted_len, int32_t* out_tokens, void* workspace,
                          size_t workspace_bytes, hipStream_t s) {
    const bool has_drafts = seq.total > seq.B;
    spec_status_t st = check_accept_common(logits, draft_tokens, rows, n_rows, seq.B, seq.K, V, has_drafts,
                                           accepted_len, out_tokens, workspace, workspace_bytes);
    if (st != SPEC_OK) return st;
    const int nr = rows ? n_rows : seq.B;
    if (nr == 0) return SPEC_OK;
    Workspace ws;
    workspace_layout(seq.B, seq.K, V, workspace, &ws);
    hipError_t e = sv::launch_softmax_stats(logits, nullptr, rows, nr, seq, V, sv::kLog2e, false, ws.stats, s);
    if (e == hipSuccess)
        e = sv::launch_accept(logits, nullptr, draft_tokens, nullptr, rows, nr, seq, V, sv::kLog2e, false,
                              pass_layout(ws.stats, nr, seq.K, V), accepted_len, out_tokens, nullptr, ws.info,
                              ws.counters, s);
    return e == hipSuccess ? SPEC_OK : hip_fail(e);
}

spec_status_t sample_impl(const float* logits, const float* draft_logits, const int32_t* draft_tokens,
                          float temperature, const uint64_t* seeds, const int32_t* rows, int n_rows, sv::SeqRows seq,
                          int V, int32_t* accepted_len, int32_t* out_tokens, float* probs_at_draft, void* workspace,
                          size_t workspace_bytes, hipStream_t s) {
    const bool has_drafts = seq.total > seq.B;
    spec_status_t st = check_accept_common(logits, draft_tokens, rows, n_rows, seq.B, seq.K, V, has_drafts,
                                           accepted_len, out_tokens, workspace, workspace_bytes);
    if (st != SPEC_OK) return st;
    if (!seeds) return SPEC_ERR_ARG;
    if (has_drafts && !draft_logits) return SPEC_ERR_ARG;
    if (!(temperature > 0.f) || !isfinite(temperature)) return SPEC_ERR_ARG;
    if (has_drafts && !aligned16(draft_logits)) return SPEC_ERR_ALIGN;
    const int nr = rows ? n_rows : seq.B;
    if (nr == 0) return SPEC_OK;
    Workspace ws;
    workspace_layout(seq.B, seq.K, V, workspace, &ws);
    const float c = sv::kLog2e / temperature;
    const float* dl = has_drafts ? draft_logits : nullptr;
    // small batches: acceptance and residual draw in one launch (their
    // latency, not their bytes, bounds the step there); every chunk
    // workgroup repeats the decision, so only while the rows to merge are few
    const bool fused = (long)nr * (2 * seq.K + 1) <= sv::kFusedAcceptMaxRows;
    hipError_t e = sv::launch_softmax_stats(logits, dl, rows, nr, seq, V, c, true, ws.stats, s,
                                            fused ? ws.counters : nullptr, sv::accept_zero_ints(seq.B, nr, V));
    if (e == hipSuccess && fused) {
        e = sv::launch_accept_residual(logits, dl, draft_tokens, seeds, rows, nr, seq, V, c,
                                       pass_layout(ws.stats, nr, seq.K, V), accepted_len, out_tokens, probs_at_draft,
                                       ws.sums, ws.counters, ws.slots, poll_limit(), s);
    } else {
        if (e == hipSuccess)
            e = sv::launch_accept(logits, dl, draft_tokens, seeds, rows, nr, seq, V, c, true,
                                  pass_layout(ws.stats, nr, seq.K, V), accepted_len, out_tokens, probs_at_draft,
                                  ws.info, ws.counters, s, ws.slots, residual_slots(nr, V));
        if (e == hipSuccess)
            e = sv::launch_residual(logits, dl, nr, V, c, ws.info, ws.sums, ws.counters, ws.slots, poll_limit(), out_tokens, s);
    }
    return e == hipSuccess ? SPEC_OK : hip_fail(e);
}

// dense batch: sequence b owns target rows b*(K+1) .. b*(K+1)+K (sizes_ok has
// bounded B*(K+1) to 31 bits)
sv::SeqRows dense_rows(int B, int K) { return sv::SeqRows{nullptr, B, K, B * (K + 1)}; }

// Records per target row the fused step may write: the direct-to-LDS
// kernel's epilogue writes one per 256 vocabulary entries (it runs only for
// M > 16; the statistics pass it may fall back to writes one per 4096).
// Records the fused step keeps beyond the accept calls' workspace: at
// M <= 16 one per cooperative-kernel workgroup for each target and draft
// row, above that one per 256 vocabulary entries for each target row.
size_t step_extra_records(int B, int K, int V) {
    const size_t M = (size_t)B * (K + 1);
    if (M <= 16) return (M + (size_t)B * K) * sv::kCoopMaxRecs;
    return M * (((size_t)V + 255) / 256);
}

// The same bound for a ragged batch of B sequences with at most K drafts
// each: its total rows R lie in [B, B*(K+1)], and R <= 16 takes the
// cooperative kernel's records for R target and R - B draft rows.
size_t step_extra_records_ragged(int B, int K, int V) {
    const size_t m_max = (size_t)B * (K + 1);
    const size_t r_coop = std::min<size_t>(16, m_max);
    const size_t coop = r_coop >= (size_t)B ? (2 * r_coop - B) * sv::kCoopMaxRecs : 0;
    const size_t big = m_max > 16 ? m_max * (((size_t)V + 255) / 256) : 0;
    return std::max(coop, big);
}

// A row list as the fused step takes it: (NULL, 0) none, (NULL, B) all,
// (list, 0..B) those.
bool rows_ok(const int32_t* rows, int n, int B) { return rows ? (n >= 0 && n <= B) : (n == 0 || n == B); }

// The whole step over any batch layout: seq.total LM-head rows (hidden
// [total, H], logits [total, V]) of which each sequence's first is its
// target-only row, and seq.total - seq.B draft rows; arguments checked by
// the caller, the workspace at least the size its entry point names.
spec_status_t step_impl(const void* hidden, const void* w_lmhead, spec_dtype_t dtype, const float* draft_logits,
                        const int32_t* draft_tokens, float temperature, const uint64_t* seeds,
                        const int32_t* greedy_rows, int n_greedy, const int32_t* sampled_rows, int n_sampled,
                        sv::SeqRows seq, int V, int H, float* logits, int32_t* accepted_len, int32_t* out_tokens,
                        float* probs_at_draft, void* workspace, size_t workspace_bytes, hipStream_t s) {
    const int B = seq.B, K = seq.K;
    const int M = seq.total;                 // LM-head rows
    const int n_drf = seq.total - seq.B;     // draft rows
    Workspace ws;
    const size_t base = workspace_layout(B, K, V, workspace, &ws);
    sv::StatRec* tstats = reinterpret_cast<sv::StatRec*>(static_cast<char*>(workspace) + base);
    const float c = n_sampled > 0 ? sv::kLog2e / temperature : sv::kLog2e;
    const int ns = sampled_rows ? n_sampled : (n_sampled ? B : 0);
    const int ng = greedy_rows ? n_greedy : (n_greedy ? B : 0);
    const bool any = ng > 0 || ns > 0;
    hipError_t e = hipSuccess;

    // At M <= 16 the cooperative kernel computes the statistics of the
    // target rows as it sums each tile and those of the draft rows while its
    // first loads are in flight, one record per workgroup and row; the accept
    // kernels merge those records straight from memory.  No pass reads the
    // logits back and no statistics kernel runs.
    const float* dl = (ns > 0 && n_drf > 0) ? draft_logits : nullptr;
    const bool fused = dl && (long)ns * (2 * K + 1) <= sv::kFusedAcceptMaxRows;
    int cus = 0;
    if (any && dtype == SPEC_BF16) {
        e = num_cus(&cus);
        if (e != hipSuccess) return hip_fail(e);
        const int crec = sv::lmhead_coop_records(M, V, H, dl ? n_drf : 0, cus);
        if (crec > 0) {
            sv::StatRec* trec = tstats;                          // M x crec
            sv::StatRec* drec = tstats + (size_t)M * crec;       // n_drf x crec
            const sv::CoopStats cs{trec, dl, dl ? n_drf : 0, drec, c, fused ? ws.counters : nullptr,
                                   fused ? sv::accept_zero_ints(B, ns, V) : 0};
            e = sv::launch_lmhead_coop_stats(static_cast<const uint16_t*>(hidden),
                                             static_cast<const uint16_t*>(w_lmhead), logits, M, V, H, cus, s, cs);
            if (e == hipSuccess && ng > 0)
                e = sv::launch_accept(logits, nullptr, draft_tokens, nullptr, greedy_rows, ng, seq, V, sv::kLog2e,
                                      false, sv::RecLayout{trec, crec, true, nullptr, 0, false}, accepted_len,
                                      out_tokens, nullptr, ws.info, ws.counters, s);
            const sv::RecLayout lay{trec, crec, true, drec, crec, true};
            if (e == hipSuccess && ns > 0) {
                if (fused) {
                    e = sv::launch_accept_residual(logits, dl, draft_tokens, seeds, sampled_rows, ns, seq, V, c, lay,
                                                   accepted_len, out_tokens, probs_at_draft, ws.sums, ws.counters, ws.slots, poll_limit(), s);
                } else {
                    e = sv::launch_accept(logits, dl, draft_tokens, seeds, sampled_rows, ns, seq, V, c, true, lay,
                                          accepted_len, out_tokens, probs_at_draft, ws.info, ws.counters, s, ws.slots, residual_slots(ns, V));
                    if (e == hipSuccess)
                        e = sv::launch_residual(logits, dl, ns, V, c, ws.info, ws.sums, ws.counters, ws.slots, poll_limit(), out_tokens, s);
                }
            }
            return e == hipSuccess ? SPEC_OK : hip_fail(e);
        }
    }

    // The statistics epilogue pays where the direct-to-LDS kernel runs: it
    // removes the pass that reads the logits back, and with the loop's order
    // pinned it costs the kernel ~2%.  Its records (one per 256 vocabulary
    // entries) are merged by the accept kernels straight from memory when a
    // sequence has at most kAcceptRowsDirect rows, else folded into the
    // statistics pass's chunk records first.  Greedy and sampled rows are
    // accepted in one launch.  Elsewhere (the skinny and tiled kernels, fp32)
    // the step runs the separate calls' kernels.
    const int big_recs = dtype == SPEC_BF16 ? sv::lmhead_big_records(M, V, H) : 0;
    const bool epilogue = any && big_recs > 0;
    if (!epilogue) {
        if (dtype == SPEC_BF16) {
            e = num_cus(&cus);
            if (e == hipSuccess)
                e = sv::launch_lmhead_bf16(static_cast<const uint16_t*>(hidden),
                                           static_cast<const uint16_t*>(w_lmhead), logits, M, V, H, cus, s);
        } else {
            e = sv::launch_lmhead_f32(static_cast<const float*>(hidden), static_cast<const float*>(w_lmhead), logits,
                                      M, V, H, s);
        }
        if (e != hipSuccess) return hip_fail(e);
        spec_status_t st = SPEC_OK;
        if (ng > 0)
            st = greedy_impl(logits, draft_tokens, greedy_rows, n_greedy, seq, V, accepted_len, out_tokens,
                             workspace, workspace_bytes, s);
        if (st == SPEC_OK && ns > 0)
            st = sample_impl(logits, draft_logits, draft_tokens, temperature, seeds, sampled_rows, n_sampled, seq, V,
                             accepted_len, out_tokens, probs_at_draft, workspace, workspace_bytes, s);
        return st;
    }

    // draft-row statistics first: they do not depend on the LM head (the pass
    // also clears the completion counters a fused accept + residual needs)
    const int nc = sv::n_chunks(V);
    if (dl) e = sv::launch_softmax_stats(nullptr, dl, sampled_rows, ns, seq, V, c, true, ws.stats, s,
                                         fused ? ws.counters : nullptr, sv::accept_zero_ints(B, ns, V));
    int nrec = 0;
    if (e == hipSuccess && cus == 0) e = num_cus(&cus);
    if (e == hipSuccess)
        e = sv::launch_lmhead_bf16(static_cast<const uint16_t*>(hidden), static_cast<const uint16_t*>(w_lmhead), logits,
                                   M, V, H, cus, s, tstats, c, &nrec);
    if (e == hipSuccess && nrec != big_recs) e = hipErrorInvalidValue;   // the kernel the shape rule named
    // target chunk records after the draft slots: B*K + M rows fit the
    // statistics area, which is sized for B*(K+1) + B*K rows (M <= B*(K+1))
    const bool direct = (ns > 0 ? 2 * K + 1 : K + 1) <= sv::kAcceptRowsDirect;
    sv::StatRec* trec = ws.stats + (size_t)B * K * nc;
    if (e == hipSuccess && !direct) e = sv::launch_fold_records(tstats, nrec, M, V, c, trec, s);
    const sv::RecLayout tgt = direct ? sv::RecLayout{tstats, nrec, true, nullptr, 0, false}
                                     : sv::RecLayout{trec, nc, true, nullptr, 0, false};
    const sv::RecLayout lay{tgt.tgt, tgt.tgt_nc, true, ws.stats, nc, false};
    if (e == hipSuccess && ng > 0 && ns > 0 && !fused) {
        e = sv::launch_accept_both(logits, dl, draft_tokens, seeds, greedy_rows, ng, sampled_rows, ns, seq, V, c, tgt,
                                   lay, accepted_len, out_tokens, probs_at_draft, ws.info, ws.counters, s, ws.slots, residual_slots(ns, V));
        if (e == hipSuccess)
            e = sv::launch_residual(logits, dl, ns, V, c, ws.info, ws.sums, ws.counters, ws.slots, poll_limit(), out_tokens, s);
        return e == hipSuccess ? SPEC_OK : hip_fail(e);
    }
    if (e == hipSuccess && ng > 0)
        e = sv::launch_accept(logits, nullptr, draft_tokens, nullptr, greedy_rows, ng, seq, V, sv::kLog2e, false, tgt,
                              accepted_len, out_tokens, nullptr, ws.info, ws.counters, s);
    if (e == hipSuccess && ns > 0) {
        if (fused) {
            e = sv::launch_accept_residual(logits, dl, draft_tokens, seeds, sampled_rows, ns, seq, V, c, lay,
                                           accepted_len, out_tokens, probs_at_draft, ws.sums, ws.counters, ws.slots, poll_limit(), s);
        } else {
            e = sv::launch_accept(logits, dl, draft_tokens, seeds, sampled_rows, ns, seq, V, c, true, lay,
                                  accepted_len, out_tokens, probs_at_draft, ws.info, ws.counters, s, ws.slots, residual_slots(ns, V));
            if (e == hipSuccess)
                e = sv::launch_residual(logits, dl, ns, V, c, ws.info, ws.sums, ws.counters, ws.slots, poll_limit(), out_tokens, s);
        }
    }
    return e == hipSuccess ? SPEC_OK : hip_fail(e);
}

}  // namespace

extern "C" {

int spec_set_poll_limit(int rounds) {
    return g_poll_limit.exchange(rounds < 0 ? sv::kDefaultPollLimit : rounds, std::memory_order_relaxed);
}

spec_status_t spec_verify_logits(const void* hidden, const void* w_lmhead, spec_dtype_t dtype, float* logits, int B,
                                 int K, int V, int H, spec_stream_t stream) {
    if (!hidden || !w_lmhead || !logits) return SPEC_ERR_ARG;
    if (dtype != SPEC_BF16 && dtype != SPEC_F32) return SPEC_ERR_DTYPE;
    if (B < 1 || K < 0 || K > kMaxK || V < 1 || H < 8 || (H & 7) != 0) return SPEC_ERR_ARG;
    if ((long long)B * (K + 1) > 0x7fffffffLL) return SPEC_ERR_ARG;
    if (!aligned16(hidden) || !aligned16(w_lmhead) || !aligned16(logits)) return SPEC_ERR_ALIGN;
    const int M = B * (K + 1);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (dtype == SPEC_BF16) {
        int cus = 0;
        e = num_cus(&cus);
        if (e != hipSuccess) return hip_fail(e);
        e = sv::launch_lmhead_bf16(static_cast<const uint16_t*>(hidden), static_cast<const uint16_t*>(w_lmhead),
                                   logits, M, V, H, cus, s);
    } else {
        e = sv::launch_lmhead_f32(static_cast<const float*>(hidden), static_cast<const float*>(w_lmhead), logits, M,
                                  V, H, s);
    }
    return e == hipSuccess ? SPEC_OK : hip_fail(e);
}

spec_status_t spec_accept_greedy(const float* logits, const int32_t* draft_tokens, const int32_t* rows, int n_rows,
                                 int B, int K, int V, int32_t* accepted_len, int32_t* out_tokens, void* workspace,
                                 size_t workspace_bytes, spec_stream_t stream) {
    if (!sizes_ok(B, K, V)) return SPEC_ERR_ARG;
    return greedy_impl(logits, draft_tokens, rows, n_rows, dense_rows(B, K), V, accepted_len, out_tokens, workspace,
                       workspace_bytes, static_cast<hipStream_t>(stream));
}

spec_status_t spec_accept_sample(const float* logits, const float* draft_logits, const int32_t* draft_tokens,
                                 float temperature, const uint64_t* seeds, const int32_t* rows, int n_rows, int B,
                                 int K, int V, int32_t* accepted_len, int32_t* out_tokens, float* probs_at_draft,
                                 void* workspace, size_t workspace_bytes, spec_stream_t stream) {
    if (!sizes_ok(B, K, V)) return SPEC_ERR_ARG;
    return sample_impl(logits, draft_logits, draft_tokens, temperature, seeds, rows, n_rows, dense_rows(B, K), V,
                       accepted_len, out_tokens, probs_at_draft, workspace, workspace_bytes,
                       static_cast<hipStream_t>(stream));
}

spec_status_t spec_accept_greedy_ragged(const float* logits, const int32_t* draft_tokens, const int32_t* row_start,
                                        int total_rows, const int32_t* rows, int n_rows, int B, int K_max, int V,
                                        int32_t* accepted_len, int32_t* out_tokens, void* workspace,
                                        size_t workspace_bytes, spec_stream_t stream) {
    if (!sizes_ok(B, K_max, V)) return SPEC_ERR_ARG;
    spec_status_t st = check_ragged(row_start, total_rows, B, K_max);
    if (st != SPEC_OK) return st;
    return greedy_impl(logits, draft_tokens, rows, n_rows, sv::SeqRows{row_start, B, K_max, total_rows}, V,
                       accepted_len, out_tokens, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

spec_status_t spec_accept_sample_ragged(const float* logits, const float* draft_logits, const int32_t* draft_tokens,
                                        const int32_t* row_start, int total_rows, float temperature,
                                        const uint64_t* seeds, const int32_t* rows, int n_rows, int B, int K_max,
                                        int V, int32_t* accepted_len, int32_t* out_tokens, float* probs_at_draft,
                                        void* workspace, size_t workspace_bytes, spec_stream_t stream) {
    if (!sizes_ok(B, K_max, V)) return SPEC_ERR_ARG;
    spec_status_t st = check_ragged(row_start, total_rows, B, K_max);
    if (st != SPEC_OK) return st;
    return sample_impl(logits, draft_logits, draft_tokens, temperature, seeds, rows, n_rows,
                       sv::SeqRows{row_start, B, K_max, total_rows}, V, accepted_len, out_tokens, probs_at_draft,
                       workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

spec_status_t spec_tree_accept_greedy(const float* logits, const int32_t* parents, const int32_t* tokens,
                                      const int32_t* rows, int n_rows, int B, int N, int V, int32_t* accepted_len,
                                      int32_t* out_tokens, int32_t* out_nodes, void* workspace,
                                      size_t workspace_bytes, spec_stream_t stream) {
    spec_status_t st = check_accept_common(logits, tokens, rows, n_rows, B, N, V, N > 0, accepted_len, out_tokens,
                                           workspace, workspace_bytes);
    if (st != SPEC_OK) return st;
    if (N > 0 && !parents) return SPEC_ERR_ARG;
    const int nr = rows ? n_rows : B;
    if (nr == 0) return SPEC_OK;
    Workspace ws;
    workspace_layout(B, N, V, workspace, &ws);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = sv::launch_softmax_stats(logits, nullptr, rows, nr, dense_rows(B, N), V, sv::kLog2e, false,
                                            ws.stats, s);
    if (e == hipSuccess)
        e = sv::launch_tree_accept(parents, tokens, rows, nr, B, N, V, ws.stats, accepted_len, out_tokens, out_nodes,
                                   s);
    return e == hipSuccess ? SPEC_OK : hip_fail(e);
}

spec_status_t spec_ngram_propose(const int32_t* history, int64_t history_len, const int64_t* hist_start, int B,
                                 int max_len, int max_ngram, int n_drafts, int32_t* drafts, int32_t* draft_count,
                                 int32_t* row_start, void* workspace, size_t workspace_bytes, spec_stream_t stream) {
    if (B < 1 || max_len < 0 || max_len == 0x7fffffff || max_ngram < 1 || max_ngram > sv::kNgMaxGram ||
        n_drafts < 0 || n_drafts > sv::kNgMaxDrafts || history_len < 0)
        return SPEC_ERR_ARG;
    if (!hist_start || !draft_count || (n_drafts > 0 && !drafts) || (history_len > 0 && !history))
        return SPEC_ERR_ARG;
    if ((long long)B * sv::ngram_segments(max_len) > 0x7fffffffLL) return SPEC_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(hist_start) & 7u) != 0) return SPEC_ERR_ALIGN;
    if (!workspace || workspace_bytes < spec_ngram_workspace_bytes(B, max_len)) return SPEC_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 7u) != 0) return SPEC_ERR_ALIGN;
    hipError_t e = sv::launch_ngram(history, history_len, hist_start, B, max_len, max_ngram, n_drafts, drafts,
                                    draft_count,
                                    row_start, static_cast<unsigned long long*>(workspace),
                                    static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SPEC_OK : hip_fail(e);
}

size_t spec_ngram_workspace_bytes(int B, int max_len) {
    if (B < 1 || max_len < 0 || max_len == 0x7fffffff) return 0;
    const size_t segs = (size_t)std::max(1, sv::ngram_segments(max_len));
    return align256((size_t)B * segs * sizeof(unsigned long long));
}

spec_status_t spec_verify_step(const void* hidden, const void* w_lmhead, spec_dtype_t dtype,
                               const float* draft_logits, const int32_t* draft_tokens, float temperature,
                               const uint64_t* seeds, const int32_t* greedy_rows, int n_greedy,
                               const int32_t* sampled_rows, int n_sampled, int B, int K, int V, int H,
                               float* logits, int32_t* accepted_len, int32_t* out_tokens, float* probs_at_draft,
                               void* workspace, size_t workspace_bytes, spec_stream_t stream) {
    if (!hidden || !w_lmhead || !logits || !accepted_len || !out_tokens) return SPEC_ERR_ARG;
    if (dtype != SPEC_BF16 && dtype != SPEC_F32) return SPEC_ERR_DTYPE;
    if (!sizes_ok(B, K, V) || H < 8 || (H & 7) != 0) return SPEC_ERR_ARG;
    if (!rows_ok(greedy_rows, n_greedy, B) || !rows_ok(sampled_rows, n_sampled, B)) return SPEC_ERR_ARG;
    const bool any = n_greedy > 0 || n_sampled > 0;
    if (any && K > 0 && !draft_tokens) return SPEC_ERR_ARG;
    if (n_sampled > 0) {
        if (!seeds || (K > 0 && !draft_logits)) return SPEC_ERR_ARG;
        if (!(temperature > 0.f) || !isfinite(temperature)) return SPEC_ERR_ARG;
        if (K > 0 && !aligned16(draft_logits)) return SPEC_ERR_ALIGN;
    }
    if (!aligned16(hidden) || !aligned16(w_lmhead) || !aligned16(logits)) return SPEC_ERR_ALIGN;
    if (!workspace || workspace_bytes < spec_verify_step_workspace_bytes(B, K, V)) return SPEC_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SPEC_ERR_ALIGN;
    return step_impl(hidden, w_lmhead, dtype, draft_logits, draft_tokens, temperature, seeds, greedy_rows, n_greedy,
                     sampled_rows, n_sampled, dense_rows(B, K), V, H, logits, accepted_len, out_tokens, probs_at_draft,
                     workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

spec_status_t spec_verify_step_ragged(const void* hidden, const void* w_lmhead, spec_dtype_t dtype,
                                      const float* draft_logits, const int32_t* draft_tokens,
                                      const int32_t* row_start, int total_rows, float temperature,
                                      const uint64_t* seeds, const int32_t* greedy_rows, int n_greedy,
                                      const int32_t* sampled_rows, int n_sampled, int B, int K_max, int V, int H,
                                      float* logits, int32_t* accepted_len, int32_t* out_tokens,
                                      float* probs_at_draft, void* workspace, size_t workspace_bytes,
                                      spec_stream_t stream) {
    if (!hidden || !w_lmhead || !logits || !accepted_len || !out_tokens) return SPEC_ERR_ARG;
    if (dtype != SPEC_BF16 && dtype != SPEC_F32) return SPEC_ERR_DTYPE;
    if (!sizes_ok(B, K_max, V) || H < 8 || (H & 7) != 0) return SPEC_ERR_ARG;
    spec_status_t st = check_ragged(row_start, total_rows, B, K_max);
    if (st != SPEC_OK) return st;
    if (!rows_ok(greedy_rows, n_greedy, B) || !rows_ok(sampled_rows, n_sampled, B)) return SPEC_ERR_ARG;
    const bool any = n_greedy > 0 || n_sampled > 0;
    const bool has_drafts = total_rows > B;
    if (any && has_drafts && !draft_tokens) return SPEC_ERR_ARG;
    if (n_sampled > 0) {
        if (!seeds || (has_drafts && !draft_logits)) return SPEC_ERR_ARG;
        if (!(temperature > 0.f) || !isfinite(temperature)) return SPEC_ERR_ARG;
        if (has_drafts && !aligned16(draft_logits)) return SPEC_ERR_ALIGN;
    }
    if (!aligned16(hidden) || !aligned16(w_lmhead) || !aligned16(logits)) return SPEC_ERR_ALIGN;
    if (!workspace || workspace_bytes < spec_verify_step_ragged_workspace_bytes(B, K_max, V)) return SPEC_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SPEC_ERR_ALIGN;
    return step_impl(hidden, w_lmhead, dtype, draft_logits, draft_tokens, temperature, seeds, greedy_rows, n_greedy,
                     sampled_rows, n_sampled, sv::SeqRows{row_start, B, K_max, total_rows}, V, H, logits,
                     accepted_len, out_tokens, probs_at_draft, workspace, workspace_bytes,
                     static_cast<hipStream_t>(stream));
}

spec_status_t spec_verify_step_noalloc(const void* hidden, const void* w_lmhead, spec_dtype_t dtype,
                                       const float* draft_logits, const int32_t* draft_tokens, float temperature,
                                       const uint64_t* seeds, const int32_t* greedy_rows, int n_greedy,
                                       const int32_t* sampled_rows, int n_sampled, int B, int K, int V, int H,
                                       float* logits, int32_t* accepted_len, int32_t* out_tokens,
                                       float* probs_at_draft, spec_stream_t stream) {
    const size_t need = spec_verify_step_workspace_bytes(B, K, V);
    if (need == 0) return SPEC_ERR_ARG;
    if (need > kNoAllocScratchBytes) {
        g_detail = "spec_verify_step_noalloc: these sizes need more than the 64 MiB of scratch the library holds "
                   "per GPU (spec_verify_step_workspace_bytes(B, K, V) > 67108864); use spec_verify_step";
        return SPEC_ERR_WORKSPACE;
    }
    void* ws = nullptr;
    hipError_t e = scratch_ptr(&ws);
    if (e != hipSuccess) return hip_fail(e);
    return spec_verify_step(hidden, w_lmhead, dtype, draft_logits, draft_tokens, temperature, seeds, greedy_rows,
                            n_greedy, sampled_rows, n_sampled, B, K, V, H, logits, accepted_len, out_tokens,
                            probs_at_draft, ws, kNoAllocScratchBytes, stream);
}

spec_status_t spec_tree_verify_step(const void* hidden, const void* w_lmhead, spec_dtype_t dtype,
                                    const int32_t* parents, const int32_t* tokens, const int32_t* rows, int n_rows,
                                    int B, int N, int V, int H, float* logits, int32_t* accepted_len,
                                    int32_t* out_tokens, int32_t* out_nodes, void* workspace,
                                    size_t workspace_bytes, spec_stream_t stream) {
    if (!hidden || !w_lmhead || !logits || !accepted_len || !out_tokens) return SPEC_ERR_ARG;
    if (dtype != SPEC_BF16 && dtype != SPEC_F32) return SPEC_ERR_DTYPE;
    if (!sizes_ok(B, N, V) || H < 8 || (H & 7) != 0) return SPEC_ERR_ARG;
    if (rows && (n_rows < 0 || n_rows > B)) return SPEC_ERR_ARG;
    if (N > 0 && (!parents || !tokens)) return SPEC_ERR_ARG;
    if (!aligned16(hidden) || !aligned16(w_lmhead) || !aligned16(logits)) return SPEC_ERR_ALIGN;
    if (!workspace || workspace_bytes < spec_verify_step_workspace_bytes(B, N, V)) return SPEC_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SPEC_ERR_ALIGN;

    const int M = B * (N + 1);
    const int nr = rows ? n_rows : B;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Workspace ws;
    const size_t base = workspace_layout(B, N, V, workspace, &ws);
    sv::StatRec* tstats = reinterpret_cast<sv::StatRec*>(static_cast<char*>(workspace) + base);
    hipError_t e = hipSuccess;
    // The tree rule needs each row's argmax only, and the bf16 LM-head kernels
    // that compute statistics on the side give it without a pass over the
    // logits: the cooperative kernel's records (one per workgroup and row),
    // or the direct-to-LDS epilogue's (one per 256 entries), folded into
    // 4096-entry chunk records; both by row.
    if (dtype == SPEC_BF16 && nr > 0) {
        int cus = 0;
        e = num_cus(&cus);
        if (e != hipSuccess) return hip_fail(e);
        const int crec = sv::lmhead_coop_records(M, V, H, 0, cus);
        if (crec > 0) {
            const sv::CoopStats cs{tstats, nullptr, 0, nullptr, sv::kLog2e, nullptr, 0};
            e = sv::launch_lmhead_coop_stats(static_cast<const uint16_t*>(hidden),
                                             static_cast<const uint16_t*>(w_lmhead), logits, M, V, H, cus, s, cs);
            if (e == hipSuccess)
                e = sv::launch_tree_accept(parents, tokens, rows, nr, B, N, V, tstats, accepted_len, out_tokens,
                                           out_nodes, s, crec, true);
            return e == hipSuccess ? SPEC_OK : hip_fail(e);
        }
        const int big_recs = sv::lmhead_big_records(M, V, H);
        if (big_recs > 0) {
            int nrec = 0;
            e = sv::launch_lmhead_bf16(static_cast<const uint16_t*>(hidden), static_cast<const uint16_t*>(w_lmhead),
                                       logits, M, V, H, cus, s, tstats, sv::kLog2e, &nrec);
            if (e == hipSuccess && nrec != big_recs) e = hipErrorInvalidValue;   // the kernel the shape rule named
            if (e == hipSuccess) e = sv::launch_fold_records(tstats, nrec, M, V, sv::kLog2e, ws.stats, s);
            if (e == hipSuccess)
                e = sv::launch_tree_accept(parents, tokens, rows, nr, B, N, V, ws.stats, accepted_len, out_tokens,
                                           out_nodes, s, 0, true);
            return e == hipSuccess ? SPEC_OK : hip_fail(e);
        }
    }
    // elsewhere (other hidden sizes, fp32, no rows): the separate calls' kernels
    spec_status_t st = spec_verify_logits(hidden, w_lmhead, dtype, logits, B, N, V, H, stream);
    if (st != SPEC_OK || nr == 0) return st;
    return spec_tree_accept_greedy(logits, parents, tokens, rows, n_rows, B, N, V, accepted_len, out_tokens, out_nodes,
                                   workspace, workspace_bytes, stream);
}

size_t spec_verify_step_workspace_bytes(int B, int K, int V) {
    if (!sizes_ok(B, K, V)) return 0;
    return workspace_layout(B, K, V, nullptr, nullptr) + align256(step_extra_records(B, K, V) * sizeof(sv::StatRec));
}

size_t spec_verify_step_ragged_workspace_bytes(int B, int K_max, int V) {
    if (!sizes_ok(B, K_max, V)) return 0;
    return workspace_layout(B, K_max, V, nullptr, nullptr) +
           align256(step_extra_records_ragged(B, K_max, V) * sizeof(sv::StatRec));
}

size_t spec_workspace_bytes(int B, int K, int V) {
    if (!sizes_ok(B, K, V)) return 0;
    return workspace_layout(B, K, V, nullptr, nullptr);
}

const char* spec_status_string(spec_status_t status) {
    switch (status) {
        case SPEC_OK: return "SPEC_OK";
        case SPEC_ERR_ARG: return "SPEC_ERR_ARG: null pointer, size out of range or bad temperature";
        case SPEC_ERR_DTYPE: return "SPEC_ERR_DTYPE: unsupported element type";
        case SPEC_ERR_ALIGN: return "SPEC_ERR_ALIGN: pointer not 16-byte aligned";
        case SPEC_ERR_WORKSPACE: return "SPEC_ERR_WORKSPACE: workspace missing or too small";
        case SPEC_ERR_HIP: return "SPEC_ERR_HIP: HIP call or kernel launch failed";
        default: break;
    }
    return "unknown spec_status_t";
}

const char* spec_last_error_detail(void) { return g_detail; }

}  // extern "C"
