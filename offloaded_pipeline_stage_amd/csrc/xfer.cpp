// Transfer engine: critical-path activation copies, and parameter uploads /
// gradient downloads packed into the data-transfer windows that follow them
// (RoundPipe paper, section 4.2.1 "The Multi-Stream Architecture" and
// section 4.2.2 "Scheduling Parameter Transfers").
//
// Four copy streams (activation up/down, parameter up, gradient down) plus the
// compute stream, each copy stream on a hardware queue of its own. Every copy
// goes by DMA (hipMemcpyAsync). A copy kernel writing downloads into the
// device mapping of the pinned host buffer does use both directions of the
// link at once next to a DMA upload (about 90 GB/s against about 57 GB/s for
// DMA both ways), but its host writes slow the compute kernels beside it by
// more than that gains (see download()).
//
// Priority of activation copies is enforced by scheduling: a window of
// parameter/gradient chunks is issued only behind the completion event of the
// activation copy it is gated on. The gate is what matters: the copy engine
// serves its streams first in, first out, so an upload issued ungated ahead
// of an activation copy delays it by the whole upload, however it is chunked
// (measured: a 67 MB activation copy takes 1.2 ms alone or gated, 17 ms
// behind an ungated 0.87 GB upload in 16 MiB chunks).
#include <algorithm>
#include <numeric>

#include "ctx.h"

namespace rp {

namespace {

struct PlanChunk {
  int item;
  uint64_t off, bytes;
  int window;
};

// split oversized items, then longest-processing-time-first assignment;
// returns chunks in item order and the issue order (by decreasing size)
std::vector<PlanChunk> make_plan(const uint64_t* sizes, int n, int n_windows, uint64_t max_chunk,
                                 uint64_t align, std::vector<int>* issue_order) {
  uint64_t total = 0;
  for (int i = 0; i < n; ++i) total += sizes[i];
  const uint64_t nw = (uint64_t)std::max(n_windows, 1);
  uint64_t thresh = (total + nw - 1) / nw;
  if (max_chunk > 0) thresh = std::min(thresh, max_chunk);
  thresh = std::max<uint64_t>(thresh, 1);
  std::vector<PlanChunk> out;
  for (int i = 0; i < n; ++i) {
    const uint64_t s = sizes[i];
    if (s <= thresh) {
      out.push_back({i, 0, s, 0});
      continue;
    }
    const uint64_t nc = (s + thresh - 1) / thresh;
    uint64_t c = (s + nc - 1) / nc;
    c = (c + align - 1) / align * align;
    for (uint64_t off = 0; off < s; off += c) out.push_back({i, off, std::min(c, s - off), 0});
  }
  std::vector<int> order(out.size());
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return out[a].bytes > out[b].bytes; });
  std::vector<uint64_t> load(nw, 0);
  for (int k : order) {
    int best = 0;
    for (int w = 1; w < (int)nw; ++w)
      if (load[w] < load[best]) best = w;
    out[k].window = best;
    load[best] += out[k].bytes;
  }
  if (issue_order) *issue_order = order;
  return out;
}

}  // namespace

rp_status new_queue_stream(int device, hipStream_t* out) {
  hipDeviceProp_t prop;
  RP_HIP(hipGetDeviceProperties(&prop, device));
  std::vector<uint32_t> mask((prop.multiProcessorCount + 31) / 32, 0xffffffffu);
  RP_HIP(hipExtStreamCreateWithCUMask(out, (uint32_t)mask.size(), mask.data()));
  return RP_OK;
}

namespace {

// device -> pinned host on stream st, by DMA: activations, checkpoints and
// gradients alike. A copy kernel writing the pinned buffer's device mapping
// was measured against it for both: its host writes slowed the compute
// kernels beside it (the streamed 8B-shaped step took 83 ms with gradient
// downloads by kernel, 64 ms by DMA; the resident step's forward QKV product
// ran three times as long next to a checkpoint download by kernel), and the
// windowed micro-batch schedule ran 13% faster with activations by DMA too.
rp_status download(void* host, const void* dev, size_t bytes, hipStream_t st) {
  RP_HIP(hipMemcpyAsync(host, dev, bytes, hipMemcpyDeviceToHost, st));
  return RP_OK;
}

hipEvent_t ticket_event(rp_ctx* c, int64_t t) {
  auto it = c->ticket_ev.find(t);
  return it == c->ticket_ev.end() ? nullptr : it->second;
}

rp_status issue_window(rp_ctx* c, XWindow& win) {
  hipStream_t st = win.dir == RP_H2D ? c->w_h2d : c->g_d2h;
  if (win.gate >= 0) {
    hipEvent_t ev = ticket_event(c, win.gate);
    RP_CHECK(ev != nullptr, RP_ERR_STATE, "transfer window gated on unknown ticket %lld", (long long)win.gate);
    RP_HIP(hipStreamWaitEvent(st, ev, 0));
  }
  Slot* prev = nullptr;
  for (XChunk& ch : win.chunks) {
    Slot& s = *ch.slot;
    if (win.dir == RP_H2D) {
      if (&s != prev && s.w_consumed_valid) RP_HIP(hipStreamWaitEvent(st, s.w_consumed, 0));
      RP_HIP(hipMemcpyAsync(ch.dev, ch.host, ch.bytes, hipMemcpyHostToDevice, st));
      if (--s.w_chunks_unissued == 0) {
        if (!s.w_ready) s.w_ready = c->new_event();
        RP_HIP(hipEventRecord(s.w_ready, st));
        s.w_ready_pending = true;
      }
    } else {
      if (&s != prev && s.g_ready_valid) RP_HIP(hipStreamWaitEvent(st, s.g_ready, 0));
      RP_TRY(download(ch.host, ch.dev, ch.bytes, st));
      if (--s.g_chunks_unissued == 0) {
        if (!s.g_drained) s.g_drained = c->new_event();
        RP_HIP(hipEventRecord(s.g_drained, st));
        s.g_drained_pending = true;
      }
    }
    prev = &s;
  }
  return RP_OK;
}

rp_status release_deferred(rp_ctx* c, int64_t ticket) {
  std::vector<XWindow> keep;
  for (XWindow& w : c->deferred) {
    if (w.gate == ticket) {
      RP_TRY(issue_window(c, w));
    } else {
      keep.push_back(std::move(w));
    }
  }
  c->deferred.swap(keep);
  return RP_OK;
}

// device buffer and size of a transfer target
rp_status resolve(rp_ctx* c, const rp_xfer& it, Slot** slot, char** dev, uint64_t* cap) {
  Slot* s = nullptr;
  switch (it.target) {
    case RP_TGT_LAYER:
    case RP_TGT_LORA:
      RP_CHECK(it.id >= 0 && it.id < (int)c->layers.size() && c->layers[it.id].bound, RP_ERR_INVALID,
               "transfer: layer %d not bound", it.id);
      s = it.target == RP_TGT_LAYER ? &c->layers[it.id].base : &c->layers[it.id].lora;
      break;
    case RP_TGT_LMHEAD:
      RP_CHECK(it.id >= 0 && it.id < c->n_shards, RP_ERR_INVALID, "transfer: LM-head shard %d not bound", it.id);
      s = &c->shards[it.id];
      break;
    case RP_TGT_FINAL_NORM:
      RP_CHECK(c->final_norm.w != nullptr, RP_ERR_INVALID, "transfer: no final norm bound");
      s = &c->final_norm;
      break;
    default:
      set_error("transfer: unknown target %d", it.target);
      return RP_ERR_INVALID;
  }
  if (it.kind == RP_PARAM_H2D) {
    RP_CHECK(s->w != nullptr, RP_ERR_INVALID, "transfer: target has no weight buffer");
    *dev = (char*)s->w;
    *cap = s->w_bytes;
  } else if (it.kind == RP_GRAD_D2H || it.kind == RP_GRAD_D2H_BF16) {
    RP_CHECK(s->g != nullptr, RP_ERR_INVALID, "transfer: target has no gradient buffer");
    *dev = (char*)s->g;
    *cap = s->g_bytes;
  } else {
    set_error("transfer: unknown kind %d", it.kind);
    return RP_ERR_INVALID;
  }
  *slot = s;
  return RP_OK;
}

}  // namespace

bool is_pinned_host(const void* p) {
  if (!p) return false;
  hipPointerAttribute_t a;
  hipError_t e = hipPointerGetAttributes(&a, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return a.type == hipMemoryTypeHost;
}

rp_status act_copy(rp_ctx* c, int dir, void* dst, const void* src, size_t bytes, int64_t* ticket) {
  RP_CHECK(dst && src, RP_ERR_INVALID, "act_copy: null pointer");
  RP_CHECK(dir == RP_H2D || dir == RP_D2H, RP_ERR_INVALID, "act_copy: bad direction %d", dir);
  RP_CHECK(is_pinned_host(dir == RP_H2D ? src : dst), RP_ERR_NOT_PINNED,
           "act_copy: host pointer is not pinned memory");
  const int64_t t = c->next_ticket;
  hipEvent_t& ev = c->ticket_ev[t];
  if (!ev) ev = c->new_event();
  if (dir == RP_H2D) {
    RP_HIP(hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, c->act_h2d));
    RP_HIP(hipEventRecord(ev, c->act_h2d));
    RP_HIP(hipStreamWaitEvent(c->compute, ev, 0));
  } else {
    if (!c->ev_mark) c->ev_mark = c->new_event();
    RP_HIP(hipEventRecord(c->ev_mark, c->compute));
    RP_HIP(hipStreamWaitEvent(c->act_d2h, c->ev_mark, 0));
    RP_TRY(download(dst, src, bytes, c->act_d2h));
    RP_HIP(hipEventRecord(ev, c->act_d2h));
  }
  c->next_ticket = t + 1;
  // keep the ticket table bounded: events of old tickets are recycled
  if (c->ticket_ev.size() > 256) {
    auto it = c->ticket_ev.begin();
    c->ev_free.push_back(it->second);
    c->ticket_ev.erase(it);
  }
  if (ticket) *ticket = t;
  return release_deferred(c, t);
}

rp_status wait_weights(rp_ctx* c, Slot& s) {
  RP_CHECK(s.w_chunks_unissued == 0, RP_ERR_STATE,
           "weights still deferred behind an activation ticket that was never issued");
  if (s.w_ready_pending) {
    RP_HIP(hipStreamWaitEvent(c->compute, s.w_ready, 0));
    s.w_ready_pending = false;
  }
  return RP_OK;
}

rp_status mark_consumed(rp_ctx* c, Slot& s) {
  if (!s.w_consumed) s.w_consumed = c->new_event();
  RP_HIP(hipEventRecord(s.w_consumed, c->compute));
  s.w_consumed_valid = true;
  return RP_OK;
}

rp_status wait_grad_drained(rp_ctx* c, Slot& s) {
  RP_CHECK(s.g_chunks_unissued == 0, RP_ERR_STATE,
           "gradient download still deferred behind an activation ticket that was never issued");
  if (s.g_drained_pending) {
    RP_HIP(hipStreamWaitEvent(c->compute, s.g_drained, 0));
    s.g_drained_pending = false;
  }
  return RP_OK;
}

rp_status mark_grad_ready(rp_ctx* c, Slot& s) {
  if (!s.g_ready) s.g_ready = c->new_event();
  RP_HIP(hipEventRecord(s.g_ready, c->compute));
  s.g_ready_valid = true;
  return RP_OK;
}

}  // namespace rp

using namespace rp;

extern "C" rp_status rp_xfer_plan(const uint64_t* sizes, int n_items, int n_windows, uint64_t max_chunk,
                                  uint64_t align, int cap, int32_t* item, uint64_t* offset, uint64_t* bytes,
                                  int32_t* window, int* n_chunks) {
  RP_CHECK(n_items >= 0 && (n_items == 0 || sizes), RP_ERR_INVALID, "xfer_plan: bad items");
  RP_CHECK(n_windows >= 1, RP_ERR_INVALID, "xfer_plan: n_windows must be >= 1");
  RP_CHECK(align >= 1, RP_ERR_INVALID, "xfer_plan: align must be >= 1");
  RP_CHECK(n_chunks, RP_ERR_INVALID, "xfer_plan: null n_chunks");
  std::vector<PlanChunk> p = make_plan(sizes, n_items, n_windows, max_chunk, align, nullptr);
  *n_chunks = (int)p.size();
  RP_CHECK((int)p.size() <= cap, RP_ERR_INVALID, "xfer_plan: %zu chunks exceed cap %d", p.size(), cap);
  for (size_t k = 0; k < p.size(); ++k) {
    if (item) item[k] = p[k].item;
    if (offset) offset[k] = p[k].off;
    if (bytes) bytes[k] = p[k].bytes;
    if (window) window[k] = p[k].window;
  }
  return RP_OK;
}

namespace rp {

// Window w waits for ticket gates[w] (or, with gates null, gate0 + w when
// gate0 >= 0); a negative gate means none.
rp_status weight_stream_submit(rp_ctx* c, const rp_xfer* items, int n_items, int n_windows, uint64_t max_chunk,
                               const int64_t* gates, int64_t gate0) {
  RP_CHECK(c, RP_ERR_INVALID, "null context");
  RP_CHECK(n_items >= 0 && (n_items == 0 || items), RP_ERR_INVALID, "submit: bad item list");
  RP_CHECK(n_windows >= 1 && n_windows <= 4096, RP_ERR_INVALID, "submit: n_windows out of range");
  // validate everything before enqueueing anything
  std::vector<Slot*> slots(n_items);
  std::vector<char*> devs(n_items);
  for (int i = 0; i < n_items; ++i) {
    const rp_xfer& it = items[i];
    uint64_t cap = 0;
    RP_TRY(resolve(c, it, &slots[i], &devs[i], &cap));
    RP_CHECK(it.offset <= cap && it.bytes <= cap - it.offset, RP_ERR_INVALID,
             "submit: item %d [%llu, +%llu) exceeds its buffer (%llu bytes)", i, (unsigned long long)it.offset,
             (unsigned long long)it.bytes, (unsigned long long)cap);
    RP_CHECK(it.host && is_pinned_host(it.host), RP_ERR_NOT_PINNED, "submit: item %d host pointer not pinned", i);
    if (it.kind == RP_GRAD_D2H_BF16) {
      RP_CHECK(it.offset % 32 == 0 && it.bytes % 32 == 0, RP_ERR_INVALID,
               "submit: item %d: a bf16 gradient download needs offset and bytes in multiples of 32", i);
      RP_CHECK(slots[i]->g_chunks_unissued == 0, RP_ERR_STATE,
               "submit: item %d: an earlier download of this gradient is still deferred", i);
    }
    devs[i] += it.offset;
  }
  // bf16 gradients: round each range on the compute stream, right behind the
  // work that wrote it (there it needs no compute units of its own and costs
  // the stream a few tenths of a millisecond per GB), into the buffer's bf16
  // staging copy; the DMA windows below copy from there. The staging copy is
  // rewritten only after its previous download, and the buffer's ready event
  // moves behind the conversion.
  for (int i = 0; i < n_items; ++i) {
    if (items[i].kind != RP_GRAD_D2H_BF16) continue;
    Slot& sl = *slots[i];
    if (!sl.g_stage) {
      RP_HIP(hipMalloc(&sl.g_stage, sl.g_bytes / 2 + 256));
      c->stages.push_back(sl.g_stage);
    }
    RP_TRY(wait_grad_drained(c, sl));
    RP_TRY(convert_f32_bf16((char*)sl.g_stage + items[i].offset / 2, (const char*)sl.g + items[i].offset,
                            items[i].bytes, c->compute));
    RP_TRY(mark_grad_ready(c, sl));
  }
  for (int dir = RP_H2D; dir <= RP_D2H; ++dir) {
    std::vector<int> idx;
    std::vector<uint64_t> sizes;
    for (int i = 0; i < n_items; ++i)
      if (dir == RP_H2D ? items[i].kind == RP_PARAM_H2D
                        : (items[i].kind == RP_GRAD_D2H || items[i].kind == RP_GRAD_D2H_BF16)) {
        idx.push_back(i);
        sizes.push_back(items[i].bytes);
      }
    if (idx.empty()) continue;
    std::vector<int> order;
    std::vector<PlanChunk> plan = make_plan(sizes.data(), (int)sizes.size(), n_windows, max_chunk, 256, &order);
    std::vector<XWindow> wins(n_windows);
    for (int w = 0; w < n_windows; ++w) {
      wins[w].dir = dir;
      wins[w].gate = gates ? (gates[w] < 0 ? -1 : gates[w]) : (gate0 < 0 ? -1 : gate0 + w);
    }
    for (int k : order) {
      const PlanChunk& pc = plan[k];
      const int i = idx[pc.item];
      XChunk ch;
      ch.dir = dir;
      ch.slot = slots[i];
      if (items[i].kind == RP_GRAD_D2H_BF16) {
        // the bf16 staging copy: half the offsets and bytes
        ch.dev = (char*)slots[i]->g_stage + (items[i].offset + pc.off) / 2;
        ch.host = (char*)items[i].host + pc.off / 2;
        ch.bytes = pc.bytes / 2;
      } else {
        ch.dev = devs[i] + pc.off;
        ch.host = (char*)items[i].host + pc.off;
        ch.bytes = pc.bytes;
      }
      if (dir == RP_H2D) ch.slot->w_chunks_unissued++;
      else ch.slot->g_chunks_unissued++;
      wins[pc.window].chunks.push_back(ch);
    }
    for (XWindow& w : wins) {
      if (w.chunks.empty()) continue;
      if (w.gate < 0 || w.gate < c->next_ticket) {
        RP_TRY(issue_window(c, w));
      } else {
        c->deferred.push_back(std::move(w));
      }
    }
  }
  return RP_OK;
}

rp_status act_wait(rp_ctx* c, int where, int64_t ticket) {
  RP_CHECK(ticket >= 0 && ticket < c->next_ticket, RP_ERR_STATE, "act_wait: ticket %lld not issued yet",
           (long long)ticket);
  hipEvent_t ev = ticket_event(c, ticket);
  RP_CHECK(ev != nullptr, RP_ERR_STATE, "act_wait: ticket %lld is too old (its event was recycled)",
           (long long)ticket);
  hipStream_t st = where == RP_ON_COMPUTE ? c->compute : where == RP_ON_ACT_H2D ? c->act_h2d : c->act_d2h;
  RP_HIP(hipStreamWaitEvent(st, ev, 0));
  return RP_OK;
}

}  // namespace rp

extern "C" rp_status rp_weight_stream_submit(rp_ctx* c, const rp_xfer* items, int n_items, int n_windows,
                                             uint64_t max_chunk, int64_t gate_ticket) {
  return rp::weight_stream_submit(c, items, n_items, n_windows, max_chunk, nullptr, gate_ticket);
}

extern "C" rp_status rp_weight_stream_submit_gated(rp_ctx* c, const rp_xfer* items, int n_items, int n_windows,
                                                   uint64_t max_chunk, const int64_t* gates) {
  RP_CHECK(gates != nullptr, RP_ERR_INVALID, "submit_gated: null gate list");
  return rp::weight_stream_submit(c, items, n_items, n_windows, max_chunk, gates, -1);
}
