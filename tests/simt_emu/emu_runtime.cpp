// Lane-thread runtime behind the host stand-in for <hip/hip_runtime.h>.
//
// Register layouts of the wave-level operations follow the CDNA3/CDNA4 ISA
// documentation of the instructions the kernels use:
//   v_mfma_f32_16x16x32_bf16: A row i = lane%16, k = 8*(lane/16)+e; B column
//     j = lane%16, same k; D column j = lane%16, rows 4*(lane/16)+r.
//   v_mfma_f32_32x32x16_bf16: A row i = lane%32, k = 8*(lane/32)+e; B column
//     j = lane%32, same k; D column j = lane%32, rows 8*(r/4)+4*(lane/32)+r%4.
//   ds_read_b64_tr_b16: in each 16-lane group, lane i names 4 bf16 of row i/4
//     (elements 4*(i%4)..) of a 4 x 16 block and receives its column i.
//   ds_read_b64_tr_b8: lane i names 8 bytes of row i/2 (bytes 8*(i%2)..) of an
//     8 x 16 byte block and receives its column i.
//   v_permlane16_swap(a, b): a' = rows {a0, b0, a2, b2}, b' = {a1, b1, a3, b3}
//     of the four 16-lane rows; v_permlane32_swap: a' = {a.lo, b.lo}, b' =
//     {a.hi, b.hi} of the two 32-lane halves.
#include <hip/hip_runtime.h>
#include <sanitizer/common_interface_defs.h>
#include <sys/mman.h>

#include <algorithm>
#include <atomic>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <memory>
#include <unordered_map>
#include <unordered_set>
#include <utility>
#include <vector>

thread_local EmuIdx threadIdx;
thread_local EmuIdx blockIdx;
thread_local EmuIdx gridDim;

hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t, int) {
  *value = 256;
  return hipSuccess;
}
hipError_t hipGetLastError() { return hipSuccess; }

// Minimal x86-64 context switch: saves the callee-saved registers on the
// current stack, stores the stack pointer to *save and resumes `to`.
extern "C" void emu_ctx_switch(void** save, void* to);
asm(R"(
  .text
  .globl emu_ctx_switch
  .type emu_ctx_switch,@function
emu_ctx_switch:
  pushq %rbp
  pushq %rbx
  pushq %r12
  pushq %r13
  pushq %r14
  pushq %r15
  movq %rsp, (%rdi)
  movq %rsi, %rsp
  popq %r15
  popq %r14
  popq %r13
  popq %r12
  popq %rbx
  popq %rbp
  ret
  .size emu_ctx_switch, .-emu_ctx_switch
)");

namespace emu {
namespace {

constexpr int kLdsLimit = 160 * 1024;      // LDS bytes of one CU
constexpr int kMaxWaves = 16;              // waves of a 1024-thread workgroup
constexpr size_t kStackBytes = 512 * 1024;  // per lane fiber

[[noreturn]] void fail(const char* what) {
  std::fprintf(stderr, "simt-emu: %s (block %u, thread %u)\n", what, blockIdx.x, threadIdx.x);
  std::fflush(stderr);
  std::abort();
}

struct Wave;
struct Barrier {
  int n = 0, count = 0;
  unsigned gen = 0;
  Wave* owner = nullptr;   // the wave of a wave rendezvous (null: the workgroup barrier)
};

struct Access {
  const unsigned char* addr;
  int bytes;
  bool write;
};

struct Wave {
  Barrier bar;
  // operands of a wave operation, lane by lane; two sets used in turn, so a
  // lane may write the next operation's operands while others still read
  // this one's (it can reach the next operation only after every lane has
  // arrived at, and so finished reading, this one)
  alignas(64) unsigned char slot[2][64][128];
  std::vector<Access> trace[64];   // LDS accesses per lane since the last analysis
};

struct Pending {
  unsigned char* dst;
  unsigned char data[16];
  int n;
};

struct Fiber {
  void* sp = nullptr;
  unsigned char* stack = nullptr;   // mapping incl. one guard page
  int tid = 0, lane = 0;
  Wave* wave = nullptr;
  Barrier* wait_bar = nullptr;
  unsigned wait_gen = 0;
  const int* wait_flag = nullptr;   // blocked until *wait_flag >= wait_target
  int wait_target = 0;
  unsigned ops = 0;                 // wave operations so far (selects the slot set)
  bool done = false;
  std::deque<Pending> dma;
  // race detector (EMU_LDS_RACE): this lane's vector clock over the waves of
  // the workgroup, and its copies not yet waited for (address, size)
  uint32_t vc[kMaxWaves] = {};
  std::deque<std::pair<uintptr_t, int>> race_dma;
};

struct Sched {
  void* sp = nullptr;
  const void* bottom = nullptr;
  size_t size = 0;
  Fiber* cur = nullptr;
  Barrier block_bar;
  std::vector<std::unique_ptr<Wave>> waves;
  Fiber* fibers = nullptr;   // the workgroup's lanes
  int nfib = 0;
  void (*body)(void*) = nullptr;
  void* arg = nullptr;
};
Sched S;

std::atomic<const unsigned char*> lds_base{nullptr};

void apply(const Pending& p) { std::memcpy(p.dst, p.data, p.n); }

// EMU_SCHED=drift runs each wave alone until it blocks at a workgroup barrier
// (waves drift apart as far as the kernel's synchronisation allows);
// EMU_SCHED=random visits the waves in a shuffled order every sweep and lets
// each take one to four wave operations (seeded by EMU_SEED), so waves get
// ahead of one another by varying, reproducible amounts; the default
// interleaves the waves one wave operation at a time.
bool drift_schedule() {
  static const bool v = [] {
    const char* e = std::getenv("EMU_SCHED");
    return e && std::strcmp(e, "drift") == 0;
  }();
  return v;
}
bool random_schedule() {
  static const bool v = [] {
    const char* e = std::getenv("EMU_SCHED");
    return e && std::strcmp(e, "random") == 0;
  }();
  return v;
}
// splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014): the schedule's random stream
uint64_t next_random() {
  static uint64_t state = [] {
    const char* e = std::getenv("EMU_SEED");
    return e ? std::strtoull(e, nullptr, 10) : 1ull;
  }();
  uint64_t z = (state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

void yield_to_scheduler(bool finishing) {
  Fiber* f = S.cur;
  void* fake = nullptr;
  __sanitizer_start_switch_fiber(finishing ? nullptr : &fake, S.bottom, S.size);
  emu_ctx_switch(&f->sp, S.sp);
  __sanitizer_finish_switch_fiber(fake, &S.bottom, &S.size);
}

bool lds_tracing();
void lds_analyze(Wave& w);

// ---- LDS race detector (EMU_LDS_RACE set, in LDS-trace builds).  Each wave
// is one thread of a happens-before model (its lanes run in program order on
// the GPU): a lane carries a vector clock over the workgroup's waves, which
// the workgroup barrier joins over all lanes, a published LDS word hands
// over (release at lds_publish, acquire when a wait sees the value) and a
// wave's own entry advances at each of those points.  Every traced LDS load
// and store, transposing read and HBM -> LDS copy is checked per dword
// against the last write and the reads since it: an access of another wave
// that the accessing lane's clock does not order before it is a race (read
// after write, write after write, write after read), whatever the schedule
// happened to do.  A copy counts as written when the issuing wave waits for
// it (vmcnt), and any access to its destination while it is in flight is a
// race, also by the issuing wave.  The first race stops the run.  Accesses
// outside the decode kernels' LDS array (the tree merge and prefill attention
// kernels' shared arrays) are tracked by address.
bool race_checking() {
  static const bool v = [] {
    if (!std::getenv("EMU_LDS_RACE")) return false;
#ifndef EMU_LDS_TRACE
    fail("EMU_LDS_RACE needs the LDS-trace build");
#endif
    return true;
  }();
  return v;
}

struct RaceCell {
  uint32_t gen = 0;        // workgroup the state belongs to (else: untouched)
  int writer = -1;         // wave of the last write, -1 if none
  int in_flight = 0;       // copies into the dword not yet waited for
  uint32_t wepoch = 0;     // the writer's epoch at that write (or at the wait)
  uint32_t reads[kMaxWaves] = {};   // each wave's latest read epoch since it
};
std::vector<RaceCell> race_cells(kLdsLimit / 4);    // the decode kernels' LDS array
std::unordered_map<uintptr_t, RaceCell> race_other;  // other kernels' shared arrays
uint32_t race_gen = 0;
struct FlagRelease {
  const int* p;
  int value;
  uint32_t vc[kMaxWaves];
};
std::vector<FlagRelease> race_flags;   // this workgroup's publishes, in order

int race_waves() { return int(S.waves.size()); }

// the LDS byte offset of an address in the decode kernels' LDS array, or -1
long lds_offset_of(uintptr_t a) {
  const uintptr_t b = reinterpret_cast<uintptr_t>(lds_base.load());
  return (b && a >= b && a < b + kLdsLimit) ? long(a - b) : -1;
}

// the state of the dword at address 4 * dword
RaceCell& race_cell(uintptr_t dword) {
  const long off = lds_offset_of(4 * dword);
  RaceCell& c = off >= 0 ? race_cells[off / 4] : race_other[dword];
  if (c.gen != race_gen) c = RaceCell{race_gen};
  return c;
}

[[noreturn]] void race_report(const char* kind, uintptr_t dword, int other, uint32_t epoch) {
  const Fiber& f = *S.cur;
  char where[64];
  const long off = lds_offset_of(4 * dword);
  if (off >= 0) std::snprintf(where, sizeof where, "LDS byte %ld", off);
  else std::snprintf(where, sizeof where, "shared address %#lx", (unsigned long)(4 * dword));
  std::fprintf(stderr,
               "simt-emu: LDS race (%s) at %s: wave %d lane %d has seen wave %d up to epoch %u, "
               "which accessed the dword at epoch %u\n",
               kind, where, f.tid >> 6, f.lane, other, other >= 0 ? f.vc[other] : 0u, epoch);
  fail("LDS race");
}

// kind: 0 load, 1 store, 2 copy issued
void race_access(const void* p, int bytes, int kind) {
  Fiber& f = *S.cur;
  const int u = f.tid >> 6;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  for (uintptr_t d = a / 4; d <= (a + uintptr_t(bytes) - 1) / 4; ++d) {
    RaceCell& c = race_cell(d);
    if (c.in_flight)
      race_report(kind == 0 ? "read of a copy in flight" : "write over a copy in flight", d,
                  c.writer, c.wepoch);
    if (c.writer >= 0 && c.writer != u && f.vc[c.writer] < c.wepoch)
      race_report(kind == 0 ? "read after write" : "write after write", d, c.writer, c.wepoch);
    if (kind == 0) {
      c.reads[u] = std::max(c.reads[u], f.vc[u]);
      continue;
    }
    for (int x = 0; x < race_waves(); ++x)
      if (x != u && c.reads[x] > f.vc[x]) race_report("write after read", d, x, c.reads[x]);
    c.writer = u;
    c.wepoch = f.vc[u];
    c.in_flight = kind == 2;
    std::fill(std::begin(c.reads), std::end(c.reads), 0u);
  }
}

// the issuing lane's wait for a copy: from here on it counts as written
void race_copy_landed(uintptr_t a, int bytes) {
  Fiber& f = *S.cur;
  for (uintptr_t d = a / 4; d <= (a + uintptr_t(bytes) - 1) / 4; ++d) {
    RaceCell& c = race_cell(d);
    c.in_flight = 0;
    c.wepoch = f.vc[f.tid >> 6];
  }
}

// the workgroup barrier opens: every lane leaves with the join of all
// lanes' clocks, its own wave's entry advanced
void race_barrier() {
  uint32_t j[kMaxWaves] = {};
  for (int t = 0; t < S.nfib; ++t)
    for (int w = 0; w < kMaxWaves; ++w) j[w] = std::max(j[w], S.fibers[t].vc[w]);
  for (int t = 0; t < S.nfib; ++t) {
    std::memcpy(S.fibers[t].vc, j, sizeof j);
    ++S.fibers[t].vc[t >> 6];
  }
}

// a wave publishes `value` at p (every lane is at the publish): the first
// lane to store it records the join of the wave's clocks
void race_release(const int* p, int value) {
  for (auto it = race_flags.rbegin(); it != race_flags.rend(); ++it)
    if (it->p == p) {
      if (it->value == value) return;
      break;
    }
  FlagRelease r{p, value, {}};
  const int w0 = 64 * (S.cur->tid >> 6);
  for (int t = w0; t < w0 + 64; ++t)
    for (int w = 0; w < kMaxWaves; ++w) r.vc[w] = std::max(r.vc[w], S.fibers[t].vc[w]);
  race_flags.push_back(r);
}

// a lane's wait saw the word at p: it acquires the publish that stored it
void race_acquire(const int* p) {
  const int v = *static_cast<const volatile int*>(p);
  for (auto it = race_flags.rbegin(); it != race_flags.rend(); ++it)
    if (it->p == p && it->value == v) {
      for (int w = 0; w < kMaxWaves; ++w) S.cur->vc[w] = std::max(S.cur->vc[w], it->vc[w]);
      return;
    }
}

void wait_on(Barrier& b) {
  const unsigned g = b.gen;
  if (++b.count == b.n) {
    // every lane of the wave (or workgroup) is here: none touches the LDS
    // until the rendezvous opens, so a wave's traced accesses line up
    if (b.owner && lds_tracing()) lds_analyze(*b.owner);
    if (!b.owner && race_checking()) race_barrier();
    b.count = 0;
    ++b.gen;
    return;
  }
  S.cur->wait_bar = &b;
  S.cur->wait_gen = g;
  yield_to_scheduler(false);
}

extern "C" void emu_fiber_entry() {
  __sanitizer_finish_switch_fiber(nullptr, &S.bottom, &S.size);
  Fiber* f = S.cur;
  S.body(S.arg);
  for (const Pending& p : f->dma) apply(p);   // the end of the program waits
  f->dma.clear();
  f->done = true;
  yield_to_scheduler(true);
  fail("finished fiber resumed");
}

// ---- LDS bank model (EMU_LDS_TRACE builds).  An instruction's lanes are
// served in groups that together move one row of the banks (banks x 4
// bytes: 8 lanes of 16 bytes with 32 banks, 16 with 64, and so on); within a
// group, every distinct dword maps to bank (address / 4) mod banks, and a
// bank holding d distinct dwords costs d - 1 extra cycles (the same dword for
// several lanes is a broadcast).  EMU_LDS_BANKS sets the bank count (64 by
// default); EMU_LDS_STATS names a file the totals are written to at exit.
struct LdsStat {
  long long instructions = 0, groups = 0, extra = 0, worst = 0;
};
struct LdsStats {
  LdsStat kind[2][5][2];   // [write][log2(bytes / 4) .. tr16 = 4][ignored]
  long long unaligned = 0;
  long long dma_lane_bytes = 0;            // bytes the HBM -> LDS copies read, lane by lane
  std::unordered_set<uintptr_t> dma_lines; // distinct 128-byte lines they read
} lds_stats;

bool lds_tracing() {
  static const bool v = std::getenv("EMU_LDS_STATS") != nullptr;
  return v;
}

int lds_banks() {
  static const int v = [] {
    const char* e = std::getenv("EMU_LDS_BANKS");
    return e ? std::atoi(e) : 64;
  }();
  return v;
}

void lds_write_stats() {
  const char* path = std::getenv("EMU_LDS_STATS");
  if (!path) return;
  FILE* f = std::fopen(path, "w");
  if (!f) return;
  static const char* names[5] = {"b32", "b64", "b128", "b256", "tr16_b64"};
  std::fprintf(f, "{\"banks\": %d, \"unaligned\": %lld, \"dma_lane_bytes\": %lld, "
               "\"dma_lines\": %zu", lds_banks(), lds_stats.unaligned, lds_stats.dma_lane_bytes,
               lds_stats.dma_lines.size());
  for (int w = 0; w < 2; ++w)
    for (int k = 0; k < 5; ++k) {
      const LdsStat& st = lds_stats.kind[w][k][0];
      if (!st.instructions) continue;
      std::fprintf(f, ", \"%s_%s\": [%lld, %lld, %lld, %lld]", w ? "write" : "read", names[k],
                   st.instructions, st.groups, st.extra, st.worst);
    }
  std::fprintf(f, "}\n");
  std::fclose(f);
}

void lds_stats_at_exit() {
  static bool registered = false;
  if (!registered) {
    registered = true;
    std::atexit(lds_write_stats);
  }
}

// Score one instruction: per-lane start addresses (nullptr: lane inactive).
void lds_score(const unsigned char* const* addr, int bytes, bool write, int kind) {
  const unsigned char* base = lds_base.load();
  if (!base) return;
  lds_stats_at_exit();
  const int banks = lds_banks();
  const int per_group = std::max(1, banks * 4 / bytes);
  LdsStat& st = lds_stats.kind[write][kind][0];
  ++st.instructions;
  for (int g0 = 0; g0 < 64; g0 += per_group) {
    std::vector<std::vector<long>> dwords(banks);
    bool any = false;
    for (int l = g0; l < g0 + per_group && l < 64; ++l) {
      if (!addr[l]) continue;
      any = true;
      const long off = long(addr[l] - base);
      for (int d = 0; d < bytes / 4; ++d) {
        const long dw = off / 4 + d;
        auto& v = dwords[dw % banks];
        if (std::find(v.begin(), v.end(), dw) == v.end()) v.push_back(dw);
      }
    }
    if (!any) continue;
    ++st.groups;
    long long degree = 1;
    for (auto& v : dwords) degree = std::max<long long>(degree, (long long)v.size());
    st.extra += degree - 1;
    st.worst = std::max(st.worst, degree);
  }
}

// Line up the lanes' traced accesses (the k-th of every lane is one
// instruction) and score them; then clear the traces.
void lds_analyze(Wave& w) {
  size_t n = 0;
  for (auto& t : w.trace) n = std::max(n, t.size());
  for (size_t k = 0; k < n; ++k) {
    const unsigned char* addr[64] = {};
    int bytes = -1;
    bool write = false, ok = true;
    for (int l = 0; l < 64; ++l) {
      if (k >= w.trace[l].size()) continue;
      const Access& a = w.trace[l][k];
      if (bytes < 0) {
        bytes = a.bytes;
        write = a.write;
      } else if (a.bytes != bytes || a.write != write) {
        ok = false;
      }
      addr[l] = a.addr;
    }
    if (!ok || (bytes != 4 && bytes != 8 && bytes != 16 && bytes != 32)) {
      ++lds_stats.unaligned;
      continue;
    }
    const int kind = bytes == 4 ? 0 : bytes == 8 ? 1 : bytes == 16 ? 2 : 3;
    lds_score(addr, bytes, write, kind);
  }
  for (auto& t : w.trace) t.clear();
}

template <typename T, typename F>
auto wave_op(const T& in, F&& f) {
  static_assert(sizeof(T) <= sizeof(Wave::slot[0][0]), "slot");
  Fiber& me = *S.cur;
  Wave& w = *me.wave;
  const int set = int(me.ops++ & 1u);
  std::memcpy(w.slot[set][me.lane], &in, sizeof(T));
  wait_on(w.bar);
  auto get = [&](int l) {
    T x;
    std::memcpy(&x, w.slot[set][l], sizeof(T));
    return x;
  };
  return f(me.lane, get);
}


}  // namespace

void run_grid(dim3 grid, dim3 block, void (*body)(void*), void* arg) {
  const int nt = int(block.x * block.y * block.z);
  if (nt % 64 != 0) fail("block size is not a multiple of 64");
  const long page = 4096;
  std::vector<Fiber> fib(nt);
  for (Fiber& f : fib) {
    void* m = mmap(nullptr, kStackBytes + page, PROT_READ | PROT_WRITE,
                   MAP_PRIVATE | MAP_ANONYMOUS | MAP_NORESERVE, -1, 0);
    if (m == MAP_FAILED) fail("cannot map a fiber stack");
    mprotect(m, page, PROT_NONE);   // guard page below the stack
    f.stack = static_cast<unsigned char*>(m);
  }
  S.body = body;
  S.arg = arg;
  S.fibers = fib.data();
  S.nfib = nt;
  if (race_checking() && nt / 64 > kMaxWaves) fail("race detector: more waves than it tracks");
  for (unsigned bz = 0; bz < grid.z; ++bz)
    for (unsigned by = 0; by < grid.y; ++by)
      for (unsigned bx = 0; bx < grid.x; ++bx) {
        S.block_bar = Barrier{nt, 0, 0};
        ++race_gen;
        race_flags.clear();
        S.waves.clear();
        for (int w = 0; w < nt / 64; ++w) {
          S.waves.push_back(std::make_unique<Wave>());
          S.waves.back()->bar.n = 64;
          S.waves.back()->bar.owner = S.waves.back().get();
        }
        for (int t = 0; t < nt; ++t) {
          Fiber& f = fib[t];
          f.tid = t;
          f.lane = t & 63;
          f.wave = S.waves[t >> 6].get();
          f.wait_bar = nullptr;
          f.wait_flag = nullptr;
          f.ops = 0;
          f.done = false;
          f.dma.clear();
          std::fill(std::begin(f.vc), std::end(f.vc), 0u);
          f.vc[t >> 6] = 1;
          f.race_dma.clear();
          // initial frame: six zeroed callee-saved registers, then the entry
          uint64_t* top = reinterpret_cast<uint64_t*>(f.stack + page + kStackBytes);
          top -= 2;
          top[0] = reinterpret_cast<uint64_t>(&emu_fiber_entry);
          top[1] = 0;
          top -= 6;
          for (int i = 0; i < 6; ++i) top[i] = 0;
          f.sp = top;
        }
        int alive = nt;
        auto resume = [&](int t) -> bool {   // false if the lane cannot run now
          Fiber& f = fib[t];
          if (f.done) return false;
          if (f.wait_bar && f.wait_bar->gen == f.wait_gen) return false;
          if (f.wait_flag && *static_cast<const volatile int*>(f.wait_flag) < f.wait_target)
            return false;
          f.wait_bar = nullptr;
          f.wait_flag = nullptr;
          threadIdx = EmuIdx{unsigned(t), 0u, 0u};
          blockIdx = EmuIdx{bx, by, bz};
          gridDim = EmuIdx{grid.x, grid.y, grid.z};
          S.cur = &f;
          void* fake = nullptr;
          __sanitizer_start_switch_fiber(&fake, f.stack + page, kStackBytes);
          emu_ctx_switch(&S.sp, f.sp);
          __sanitizer_finish_switch_fiber(fake, nullptr, nullptr);
          if (f.done) --alive;
          return true;
        };
        const int nw = nt / 64;
        unsigned rot = 0;
        while (alive > 0) {
          bool progressed = false;
          if (drift_schedule()) {
            // one wave at a time, run until it can go no further (it waits
            // at a workgroup barrier or has finished); start with a rotating
            // wave so that every wave gets ahead of the others in turn
            for (int k = 0; k < nw; ++k) {
              const int w = int((rot + k) % nw);
              for (bool moved = true; moved;) {
                moved = false;
                for (int t = 64 * w; t < 64 * w + 64; ++t) moved |= resume(t);
                progressed |= moved;
              }
            }
            ++rot;
          } else if (random_schedule()) {
            std::vector<int> order(nw);
            for (int w = 0; w < nw; ++w) order[w] = w;
            for (int w = nw - 1; w > 0; --w) std::swap(order[w], order[next_random() % (w + 1)]);
            for (int w : order) {
              const int steps = 1 + int(next_random() % 4);
              for (int k = 0; k < steps; ++k)
                for (int t = 64 * w; t < 64 * w + 64; ++t) progressed |= resume(t);
            }
          } else {
            for (int t = 0; t < nt; ++t) progressed |= resume(t);
          }
          if (!progressed)
            fail("deadlock: every live lane waits at a barrier no lane can complete, or for an "
                 "LDS word no lane raises");
        }
        if (lds_tracing())
          for (auto& w : S.waves) lds_analyze(*w);
      }
  for (Fiber& f : fib) munmap(f.stack, kStackBytes + page);
}

uint32_t lds_address(const void* p) {
  const unsigned char* c = static_cast<const unsigned char*>(p);
  const unsigned char* expected = nullptr;
  lds_base.compare_exchange_strong(expected, c);
  const unsigned char* b = lds_base.load();
  if (c < b || c - b >= kLdsLimit) fail("LDS address outside the shared array");
  return uint32_t(c - b);
}

// EMU_DMA_LAND=issue lands every copy at once (a copy into a stage that
// another wave still reads then corrupts that read: write-after-read races);
// the default lands copies at the issuing wave's vmcnt wait (a read before
// the wait sees stale data: read-after-write races).
bool land_at_issue() {
  static const bool v = [] {
    const char* e = std::getenv("EMU_DMA_LAND");
    return e && std::strcmp(e, "issue") == 0;
  }();
  return v;
}

void lds_dma(uint32_t lds, int voff, const void* sbase, int bytes) {
  const unsigned char* b = lds_base.load();
  if (!b) fail("LDS copy before any LDS address was taken");
  const uint64_t off = uint64_t(lds) + uint64_t(bytes) * S.cur->lane;
  if (off + bytes > uint64_t(kLdsLimit)) fail("LDS copy destination beyond the LDS size");
  Pending p;
  p.dst = const_cast<unsigned char*>(b) + off;
  p.n = bytes;
  std::memcpy(p.data, static_cast<const unsigned char*>(sbase) + voff, bytes);   // checked read
  if (lds_tracing()) {
    lds_stats_at_exit();
    const uintptr_t a = reinterpret_cast<uintptr_t>(sbase) + uintptr_t(voff);
    lds_stats.dma_lane_bytes += bytes;
    for (uintptr_t line = a / 128; line <= (a + bytes - 1) / 128; ++line)
      lds_stats.dma_lines.insert(line);
  }
  if (race_checking()) {
    race_access(p.dst, bytes, 2);
    S.cur->race_dma.emplace_back(reinterpret_cast<uintptr_t>(p.dst), bytes);
  }
  if (land_at_issue()) apply(p);
  else S.cur->dma.push_back(p);
}

// s_waitcnt is per wave: every lane's copies land before any lane goes on.
void vm_wait(int n) {
  auto& q = S.cur->dma;
  while (int(q.size()) > n) {
    apply(q.front());
    q.pop_front();
  }
  auto& r = S.cur->race_dma;
  while (int(r.size()) > n) {
    race_copy_landed(r.front().first, r.front().second);
    r.pop_front();
  }
  wait_on(S.cur->wave->bar);
}

void block_barrier() { wait_on(S.block_bar); }

void lds_trace_access(const void* p, int bytes, bool write) {
  if (lds_tracing()) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    if (lds_offset_of(a) < 0 || lds_offset_of(a + bytes - 1) < 0)
      fail("LDS access outside the LDS");
    S.cur->wave->trace[S.cur->lane].push_back(
        Access{static_cast<const unsigned char*>(p), bytes, write});
  }
  if (race_checking()) race_access(p, bytes, write ? 1 : 0);
}

// Publishing an LDS word is a wave operation: every lane of the wave has
// made its earlier LDS writes before any lane stores the word.
void flag_publish(int* p, int value) {
  const unsigned char* b = lds_base.load();
  const unsigned char* c = reinterpret_cast<const unsigned char*>(p);
  if (!b || c < b || c + sizeof(int) > b + kLdsLimit) fail("flag store outside the LDS");
  wait_on(S.cur->wave->bar);
  if (race_checking()) race_release(p, value);
  *static_cast<volatile int*>(p) = value;
  if (race_checking()) ++S.cur->vc[S.cur->tid >> 6];
}

// A lane waiting for an LDS word another wave publishes is not resumed until
// the word reaches the target (so under EMU_SCHED=drift the other waves run
// meanwhile), and a wait that nothing can end is reported as a deadlock.
void flag_wait(const int* p, int target) {
  const unsigned char* b = lds_base.load();
  const unsigned char* c = reinterpret_cast<const unsigned char*>(p);
  if (!b || c < b || c + sizeof(int) > b + kLdsLimit) fail("flag wait outside the LDS");
  if (*static_cast<const volatile int*>(p) < target) {
    S.cur->wait_flag = p;
    S.cur->wait_target = target;
    yield_to_scheduler(false);
  }
  if (race_checking()) race_acquire(p);
}

uint32_t readfirstlane(uint32_t v) {
  return wave_op(v, [](int, auto get) { return get(0); });
}
uint32_t readlane(uint32_t v, int lane) {
  if (lane < 0 || lane > 63) fail("readlane of a lane outside the wave");
  return wave_op(v, [lane](int, auto get) { return get(lane); });
}

int shfl_xor(int v, int mask) {
  return wave_op(v, [mask](int l, auto get) { return get((l ^ mask) & 63); });
}
float shfl_xor(float v, int mask) {
  return wave_op(v, [mask](int l, auto get) { return get((l ^ mask) & 63); });
}

int any(int pred) {
  return wave_op(pred != 0, [](int, auto get) {
    for (int l = 0; l < 64; ++l)
      if (get(l)) return 1;
    return 0;
  });
}

emu_u32x2 permlane16_swap(uint32_t a, uint32_t b) {
  struct AB { uint32_t a, b; };
  return wave_op(AB{a, b}, [](int l, auto get) {
    const int row = l >> 4;
    emu_u32x2 r;
    r[0] = (row & 1) ? get(l - 16).b : get(l).a;
    r[1] = (row & 1) ? get(l).b : get(l + 16).a;
    return r;
  });
}

emu_u32x2 permlane32_swap(uint32_t a, uint32_t b) {
  struct AB { uint32_t a, b; };
  return wave_op(AB{a, b}, [](int l, auto get) {
    emu_u32x2 r;
    r[0] = l < 32 ? get(l).a : get(l - 32).b;
    r[1] = l < 32 ? get(l + 32).a : get(l).b;
    return r;
  });
}

emu_f32x4 mfma16x16x32(emu_bf16x8 a, emu_bf16x8 b, emu_f32x4 c) {
  struct In { emu_bf16x8 a, b; };
  const emu_f32x4 out = wave_op(In{a, b}, [](int l, auto get) {
    // the operands this lane's outputs use, each fetched once; the products
    // are summed in k order as before
    emu_f32x4 d;
    const int j = l & 15;
    emu_bf16x8 bq[4];
    for (int q = 0; q < 4; ++q) bq[q] = get(j + 16 * q).b;
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * (l >> 4) + r;
      emu_bf16x8 aq[4];
      for (int q = 0; q < 4; ++q) aq[q] = get(i + 16 * q).a;
      float s = 0.f;
      for (int k = 0; k < 32; ++k) s += float(aq[k >> 3][k & 7]) * float(bq[k >> 3][k & 7]);
      d[r] = s;
    }
    return d;
  });
  return out + c;
}

emu_f32x16 mfma32x32x16(emu_bf16x8 a, emu_bf16x8 b, emu_f32x16 c) {
  struct In { emu_bf16x8 a, b; };
  const emu_f32x16 out = wave_op(In{a, b}, [](int l, auto get) {
    // the operands this lane's outputs use, each fetched once; the products
    // are summed in k order as before
    emu_f32x16 d;
    const int j = l & 31;
    const emu_bf16x8 b0 = get(j).b, b1 = get(j + 32).b;
    for (int r = 0; r < 16; ++r) {
      const int i = 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
      const emu_bf16x8 a0 = get(i).a, a1 = get(i + 32).a;
      float s = 0.f;
      for (int k = 0; k < 8; ++k) s += float(a0[k]) * float(b0[k]);
      for (int k = 0; k < 8; ++k) s += float(a1[k]) * float(b1[k]);
      d[r] = s;
    }
    return d;
  });
  return out + c;
}

emu_bf16x4 ds_read_tr16_b64(const emu_bf16x4* p) {
  if (race_checking()) race_access(p, 8, 0);
  return wave_op(p, [](int l, auto get) {
    if (l == 0 && lds_tracing()) {
      const unsigned char* addr[64];
      for (int k = 0; k < 64; ++k) addr[k] = reinterpret_cast<const unsigned char*>(get(k));
      lds_score(addr, 8, false, 4);
    }
    const int g = l >> 4, i = l & 15;
    emu_bf16x4 r;
    for (int row = 0; row < 4; ++row) {
      emu_bf16x4 v;
      std::memcpy(&v, get(16 * g + 4 * row + (i >> 2)), sizeof v);   // checked 8-byte read
      r[row] = v[i & 3];
    }
    return r;
  });
}

emu_i32x2 ds_read_tr8_b64(const emu_i32x2* p) {
  if (race_checking()) race_access(p, 8, 0);
  return wave_op(p, [](int l, auto get) {
    const int g = l >> 4, i = l & 15;
    unsigned char out[8];
    for (int row = 0; row < 8; ++row) {
      unsigned char v[8];
      std::memcpy(v, get(16 * g + 2 * row + (i >> 3)), 8);
      out[row] = v[i & 7];
    }
    emu_i32x2 r;
    std::memcpy(&r, out, 8);
    return r;
  });
}

// OCP e4m3 (FN variant: no infinities, S.1111.111 is NaN), bias 7.
static float e4m3_to_f32(unsigned v) {
  const unsigned s = (v >> 7) & 1, e = (v >> 3) & 15, m = v & 7;
  float x;
  if (e == 15 && m == 7) x = NAN;
  else if (e == 0) x = std::ldexp(float(m), -9);
  else x = std::ldexp(float(8 + m), int(e) - 10);
  return s ? -x : x;
}

// Nearest e4m3 code by search over the codes' values (monotone in the code
// for codes 0..126), ties to the even code; the sign is carried over.
uint32_t e4m3_rne(float x) {
  if (!(std::fabs(x) <= 448.f)) fail("e4m3 conversion of a value outside +-448 (or NaN)");
  const float a = std::fabs(x);
  unsigned lo = 0, hi = 126;                 // value(lo) <= a <= value(hi)
  while (hi - lo > 1) {
    const unsigned mid = (lo + hi) / 2;
    if (e4m3_to_f32(mid) <= a) lo = mid; else hi = mid;
  }
  const double dl = double(a) - e4m3_to_f32(lo), dh = double(e4m3_to_f32(hi)) - a;
  unsigned c = dl < dh ? lo : dh < dl ? hi : ((lo & 1u) ? hi : lo);
  if (a == e4m3_to_f32(hi)) c = hi;
  return c | (std::signbit(x) ? 0x80u : 0u);
}

// 16x16x64 int8: lane l supplies row (A) / column (B) l % 16 and the 16
// k-values 16 (l / 16) .. + 15, byte j of its operand being k = 16 (l / 16) + j
// (the same k order for A and B); output lane l holds rows 4 (l / 16) + r of
// column l % 16.
emu_i32x4 mfma_i8_16x16x64(emu_i32x4 a, emu_i32x4 b, emu_i32x4 c) {
  struct In { emu_i32x4 a, b; };
  const emu_i32x4 out = wave_op(In{a, b}, [](int l, auto get) {
    emu_i32x4 d;
    const int j = l & 15;
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * (l >> 4) + r;
      int32_t s = 0;
      for (int k = 0; k < 64; ++k) {
        const emu_i32x4 av = get(i + 16 * (k >> 4)).a, bv = get(j + 16 * (k >> 4)).b;
        const int8_t x = int8_t(uint32_t(av[(k & 15) >> 2]) >> (8 * (k & 3)));
        const int8_t y = int8_t(uint32_t(bv[(k & 15) >> 2]) >> (8 * (k & 3)));
        s += int32_t(x) * int32_t(y);
      }
      d[r] = s;
    }
    return d;
  });
  return out + c;
}

// 16x16x128 e4m3 x e4m3 (format code 0 for both operands) with e8m0 block
// scales: lane l supplies row / column l % 16 and k-values 32 (l / 16) .. + 31,
// byte j being k = 32 (l / 16) + j; its scale byte (2^(byte - 127)) applies to
// those 32 values of its row (A) or column (B).  Output as above.
emu_f32x4 mfma_f8_16x16x128(emu_i32x8 a, emu_i32x8 b, emu_f32x4 c, int fmt_a, int fmt_b,
                            int scale_a, int scale_b) {
  if (fmt_a != 0 || fmt_b != 0) fail("mfma f8f6f4: only e4m3 operands are modelled");
  struct In { emu_i32x8 a, b; int sa, sb; };
  const emu_f32x4 out = wave_op(In{a, b, scale_a & 0xFF, scale_b & 0xFF}, [](int l, auto get) {
    emu_f32x4 d;
    const int j = l & 15;
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * (l >> 4) + r;
      double s = 0.0;
      for (int k = 0; k < 128; ++k) {
        const In ai = get(i + 16 * (k >> 5)), bj = get(j + 16 * (k >> 5));
        const unsigned x = (uint32_t(ai.a[(k & 31) >> 2]) >> (8 * (k & 3))) & 0xFFu;
        const unsigned y = (uint32_t(bj.b[(k & 31) >> 2]) >> (8 * (k & 3))) & 0xFFu;
        s += std::ldexp(double(e4m3_to_f32(x)) * double(e4m3_to_f32(y)),
                        (ai.sa - 127) + (bj.sb - 127));
      }
      d[r] = float(s);
    }
    return d;
  });
  return out + c;
}

emu_f32x2 cvt_pk_f32_fp8(int v, bool hi) {
  const unsigned u = unsigned(v) >> (hi ? 16 : 0);
  emu_f32x2 r;
  r[0] = e4m3_to_f32(u & 0xff);
  r[1] = e4m3_to_f32((u >> 8) & 0xff);
  return r;
}

}  // namespace emu
