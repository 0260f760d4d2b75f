// Copies on the GPU's SDMA engines (the copy-engine path of the param-contiguous gather).
//
// Page "ccl: hierarchical cross-node AllGather (intra-node SDMA + inter-node RDMA) #441" moves its
// intra-node all-gather on copy engines, which leave the compute units to a concurrent GEMM.  On one
// GPU the same engines serve device-to-device copies when they are asked for explicitly: HIP's
// device-to-device copies are blit kernels on this runtime, so this file drives the engines through
// the HSA runtime (hsa_amd_memory_async_copy_on_engine with the copy forced onto SDMA).  Measured on
// an MI355X: 14 engines (mask 0xfffc), about 51 GB/s of copy each plus about 15 us per copy command
// (1.1 TB/s of read + write bytes together on 4 MiB copies), results bit-exact, and no kernel dispatch
// in a kernel trace.  The 2-D form (hsa_amd_memory_async_copy_rect) ran at a few GB/s, so strided
// blocks go as one 1-D copy per row.

#include <hsa/hsa.h>
#include <hsa/hsa_ext_amd.h>

#include <chrono>
#include <cstdio>
#include <algorithm>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "mr_internal.h"

namespace mr {
namespace {

struct Engines {
  bool ready = false;
  hsa_status_t init_status = HSA_STATUS_SUCCESS;
  hsa_agent_t agent{};
  std::vector<uint32_t> ids;  // hsa_amd_sdma_engine_id_t bits
};

std::mutex g_mu;
std::vector<Engines> g_dev;  // per HIP device

struct Find {
  bool have_pci;  // the HIP device's PCI location is known
  uint32_t domain, bdf;
  int gpus;
  hsa_agent_t match, first, cpu;
  bool found, have_cpu;
};

hsa_status_t visit(hsa_agent_t a, void* data) {
  Find* f = static_cast<Find*>(data);
  hsa_device_type_t t;
  if (hsa_agent_get_info(a, HSA_AGENT_INFO_DEVICE, &t) != HSA_STATUS_SUCCESS) return HSA_STATUS_SUCCESS;
  if (t == HSA_DEVICE_TYPE_CPU && !f->have_cpu) {
    f->cpu = a;
    f->have_cpu = true;
  }
  if (t != HSA_DEVICE_TYPE_GPU) return HSA_STATUS_SUCCESS;
  if (f->gpus++ == 0) f->first = a;
  uint32_t bdf = 0, dom = 0;
  hsa_agent_get_info(a, static_cast<hsa_agent_info_t>(HSA_AMD_AGENT_INFO_BDFID), &bdf);
  hsa_agent_get_info(a, static_cast<hsa_agent_info_t>(HSA_AMD_AGENT_INFO_DOMAIN), &dom);
  if (std::getenv("MR_TRACE"))
    std::fprintf(stderr, "[mr] hsa gpu agent %d: domain %u bdfid %#x (hip device: domain %u bdfid %#x, known %d)\n",
                 f->gpus - 1, dom, bdf, f->domain, f->bdf, f->have_pci ? 1 : 0);
  if (!f->found && f->have_pci && (bdf >> 3) == (f->bdf >> 3) && dom == f->domain) {
    f->match = a;
    f->found = true;
  }
  return HSA_STATUS_SUCCESS;
}

// The HSA agent and SDMA engines of HIP device `dev` (found once per process).
int engines_for(int dev, Engines** out) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (static_cast<int>(g_dev.size()) <= dev) g_dev.resize(dev + 1);
  Engines& e = g_dev[dev];
  if (!e.ready) {
    e.ready = true;
    // PCI location of the HIP device, to pick its HSA agent; with one GPU agent it is that one anyway
    int bus = 0, device = 0, domain = 0;
    const bool have_pci = hipDeviceGetAttribute(&bus, hipDeviceAttributePciBusId, dev) == hipSuccess &&
                          hipDeviceGetAttribute(&device, hipDeviceAttributePciDeviceId, dev) == hipSuccess &&
                          hipDeviceGetAttribute(&domain, hipDeviceAttributePciDomainId, dev) == hipSuccess;
    if ((e.init_status = hsa_init()) == HSA_STATUS_SUCCESS) {
      Find f{have_pci, static_cast<uint32_t>(domain), static_cast<uint32_t>((bus << 8) | (device << 3)), 0, {}, {}, {},
             false, false};
      e.init_status = hsa_iterate_agents(visit, &f);
      if (e.init_status == HSA_STATUS_SUCCESS && !f.found && f.gpus == 1) {  // one GPU: it is this device
        f.match = f.first;
        f.found = true;
      }
      if (e.init_status == HSA_STATUS_SUCCESS && !f.found) e.init_status = HSA_STATUS_ERROR_INVALID_AGENT;
      uint32_t mask = 0;
      if (e.init_status == HSA_STATUS_SUCCESS) {
        // Engines for copies inside the device's own memory.  The HSA runtime of ROCm 7.2 answers this
        // query with engines 2..15 (mask 0xfffc; 0 and 1 serve host transfers); the one bundled with
        // ROCm 7.0 refuses a device-to-itself query (HSA_STATUS_ERROR_INVALID_AGENT) but answers the
        // host-to-device one with 0xffff, so that mask less engines 0 and 1 stands in for it.
        e.init_status = hsa_amd_memory_copy_engine_status(f.match, f.match, &mask);
        const hsa_status_t same = e.init_status;
        if (e.init_status != HSA_STATUS_SUCCESS && f.have_cpu) {
          uint32_t host_mask = 0;
          e.init_status = hsa_amd_memory_copy_engine_status(f.match, f.cpu, &host_mask);
          mask = host_mask & ~0x3u;
        }
        if (std::getenv("MR_TRACE"))
          std::fprintf(stderr, "[mr] sdma engines: device-local query %#x, engine mask %#x (status %#x)\n",
                       static_cast<unsigned>(same), mask, static_cast<unsigned>(e.init_status));
      }
      if (e.init_status == HSA_STATUS_SUCCESS) {
        e.agent = f.match;
        for (int i = 0; i < 32; ++i)
          if (mask & (1u << i)) e.ids.push_back(1u << i);
        if (e.ids.empty()) e.init_status = HSA_STATUS_ERROR_OUT_OF_RESOURCES;
      }
    }
  }
  *out = &e;
  return static_cast<int>(e.init_status);
}

}  // namespace

// Copies larger than this are cut so that every engine gets a share of a large gather.  Same-GPU A/B
// (alternating processes, W=8 G=4 P=64 FSDP-style splits with parameters under 1 MiB per rank on the
// kernel / one 430 MB parameter), per call: cuts at 2 MiB 736-754 / 787-809 us, 4 MiB 682-698 / 771-775,
// 8 MiB 664-685 / 752-759 (scheduling model below in each case).
#ifndef MR_SDMA_CHUNK_MIB
#define MR_SDMA_CHUNK_MIB 8
#endif
constexpr uint64_t kSdmaChunk = uint64_t(MR_SDMA_CHUNK_MIB) << 20;
#ifndef MR_SDMA_LPT
#define MR_SDMA_LPT 1
#endif
#ifndef MR_SDMA_QUIET
#define MR_SDMA_QUIET 1
#endif
// Scheduling model of one engine: a copy costs its bytes at kEngineBytesPerUs plus kCopyUs (each
// copy command costs an engine about 15 us beyond its bytes: 448 copies of 2 KiB to 256 KiB over 14
// engines took 15-17 us per copy per engine, and 4 MiB copies ran at about 51 GB/s past that).  Copies
// are dealt longest first to the engine that frees up first, and only each engine's last copy signals
// the waited signal (the others a quiet one: no completion interrupt per copy).  Same-GPU A/B, W=8, G=4,
// P=64 bf16, every piece on the engines (536 copies on 14 engines), per call: bytes dealt round-robin by
// bytes, every copy on the waited signal 1335 us; longest first 1196 us; quiet signals 1131 us; both
// 1080 us.  One 430 MB parameter (103 copies): 792 -> 772 us.  The fitted model (51 GB/s, 15 us)
// against the first guess (40 GB/s, 10 us), 8 MiB cuts: 664-685 against 668-685 us with the default split.
#ifndef MR_SDMA_ENGINE_BYTES_PER_US
#define MR_SDMA_ENGINE_BYTES_PER_US 51000.0
#endif
#ifndef MR_SDMA_COPY_US
#define MR_SDMA_COPY_US 15.0
#endif
constexpr double kEngineBytesPerUs = MR_SDMA_ENGINE_BYTES_PER_US;
constexpr double kCopyUs = MR_SDMA_COPY_US;

// A signal that only the engines decrement and nobody waits on (no completion interrupt): the
// completion signal of every copy but the last one on each engine.  One per device, kept for the
// process's life; 0 if the runtime gave none (then every copy signals the waited one).
uint64_t quiet_signal(int dev) {
  static std::mutex mu;
  static std::vector<uint64_t> sig;
  std::lock_guard<std::mutex> lk(mu);
  if (static_cast<int>(sig.size()) <= dev) sig.resize(dev + 1, 0);
  if (!sig[dev]) {
    hsa_signal_t q;
    if (hsa_amd_signal_create(0, 0, nullptr, HSA_AMD_SIGNAL_AMD_GPU_ONLY, &q) == HSA_STATUS_SUCCESS) sig[dev] = q.handle;
  }
  return sig[dev];
}

int sdma_copy(const CopyPiece* pieces, size_t count) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return static_cast<int>(HSA_STATUS_ERROR_INVALID_AGENT);
  Engines* e = nullptr;
  const int init = engines_for(dev, &e);
  if (init != HSA_STATUS_SUCCESS) return init;
  struct Job { const char* src; char* dst; uint64_t bytes; };
  std::vector<Job> jobs;
  for (size_t i = 0; i < count; ++i)
    for (uint64_t off = 0; off < pieces[i].bytes; off += kSdmaChunk) {
      const uint64_t len = pieces[i].bytes - off < kSdmaChunk ? pieces[i].bytes - off : kSdmaChunk;
      jobs.push_back({pieces[i].src + off, pieces[i].dst + off, len});
    }
  if (jobs.empty()) return 0;
  const bool trace = std::getenv("MR_TRACE") != nullptr;
  const auto t0 = std::chrono::steady_clock::now();
  // Longest first, each to the engine that frees up first (copies on one engine run in order).
  const size_t E = e->ids.size();
  std::vector<std::vector<size_t>> per(E);
  std::vector<double> busy(E, 0.0);
  std::vector<size_t> order(jobs.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = i;
  if (MR_SDMA_LPT)
    std::stable_sort(order.begin(), order.end(), [&](size_t a, size_t b) { return jobs[a].bytes > jobs[b].bytes; });
  for (size_t i : order) {
    size_t best = 0;
    for (size_t k = 1; k < E; ++k)
      if (busy[k] < busy[best]) best = k;
    busy[best] += static_cast<double>(jobs[i].bytes) / kEngineBytesPerUs + (MR_SDMA_LPT ? kCopyUs : 0.0);
    per[best].push_back(i);
  }
  size_t used = 0;
  for (size_t k = 0; k < E; ++k) used += per[k].empty() ? 0 : 1;
  hsa_signal_t quiet{MR_SDMA_QUIET ? quiet_signal(dev) : 0};
  // the waited signal counts the engines' last copies, or every copy without a quiet signal
  const size_t waited = quiet.handle ? used : jobs.size();
  hsa_signal_t sig;
  hsa_status_t st = hsa_signal_create(static_cast<hsa_signal_value_t>(waited), 0, nullptr, &sig);
  if (st != HSA_STATUS_SUCCESS) return static_cast<int>(st);
  // issue round-robin over the engines so that every engine starts at once
  auto issue = [&](size_t k, const Job& j, hsa_signal_t done) {
    return hsa_amd_memory_async_copy_on_engine(j.dst, e->agent, j.src, e->agent, j.bytes, 0, nullptr, done,
                                               static_cast<hsa_amd_sdma_engine_id_t>(e->ids[k]), true);
  };
  size_t pending = waited;
  std::vector<size_t> issued(E, 0);
  for (size_t r = 0; st == HSA_STATUS_SUCCESS; ++r) {
    bool any = false;
    for (size_t k = 0; k < E && st == HSA_STATUS_SUCCESS; ++k) {
      if (r >= per[k].size()) continue;
      any = true;
      const hsa_signal_t done = quiet.handle && r + 1 < per[k].size() ? quiet : sig;
      st = issue(k, jobs[per[k][r]], done);
      if (st == HSA_STATUS_SUCCESS) {
        ++issued[k];
        if (done.handle == sig.handle) --pending;
      }
    }
    if (!any) break;
  }
  if (st != HSA_STATUS_SUCCESS && quiet.handle) {
    // An engine that has copies in flight on the quiet signal but not its last one: copy its last issued
    // piece again (the same bytes) with the waited signal, so that the wait below covers that engine too.
    for (size_t k = 0; k < E; ++k)
      if (issued[k] && issued[k] < per[k].size() && issue(k, jobs[per[k][issued[k] - 1]], sig) == HSA_STATUS_SUCCESS)
        --pending;
  }
  const auto t1 = std::chrono::steady_clock::now();
  // decrements that will never come (copies not issued) are taken off before waiting for the rest
  if (pending) hsa_signal_subtract_screlease(sig, static_cast<hsa_signal_value_t>(pending));
  const hsa_signal_value_t v =
      hsa_signal_wait_scacquire(sig, HSA_SIGNAL_CONDITION_LT, 1, UINT64_MAX, HSA_WAIT_STATE_BLOCKED);
  hsa_signal_destroy(sig);
  if (trace) {
    const auto t2 = std::chrono::steady_clock::now();
    std::fprintf(stderr, "[mr] sdma: %zu copies on %zu engines, submitted in %.1f us, done after %.1f us\n", jobs.size(),
                 used, std::chrono::duration<double, std::micro>(t1 - t0).count(),
                 std::chrono::duration<double, std::micro>(t2 - t0).count());
  }
  if (st != HSA_STATUS_SUCCESS) return static_cast<int>(st);
  return v < 0 ? -1 : 0;  // a negative signal value reports a failed copy
}

int sdma_engine_count(int* status) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    *status = static_cast<int>(HSA_STATUS_ERROR_INVALID_AGENT);
    return 0;
  }
  Engines* e = nullptr;
  *status = engines_for(dev, &e);
  return *status == HSA_STATUS_SUCCESS ? static_cast<int>(e->ids.size()) : 0;
}

}  // namespace mr
