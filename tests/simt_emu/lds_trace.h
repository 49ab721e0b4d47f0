// LDS access tracing for the emulator (built only with EMU_LDS_TRACE).
//
// With it, LDS_PTR(T) is emu::LdsP<T> instead of T*: every load and store the
// decode kernels make through an LDS pointer is logged per lane, and at each
// wave rendezvous the accesses of the wave's lanes are lined up (the k-th
// access of every lane is one instruction) and scored against a model of the
// LDS banks (emu_runtime.cpp); with EMU_LDS_RACE each access is also checked
// by the runtime's happens-before race detector.  The decode kernels, the tree
// merge kernel and the prefill attention kernel use LDS_PTR.
#pragma once
#include <cstddef>

namespace emu {
void lds_trace_access(const void* p, int bytes, bool write);

template <typename T>
struct LdsRef {
  T* p;
  operator T() const {
    lds_trace_access(p, int(sizeof(T)), false);
    return *p;
  }
  const LdsRef& operator=(const T& v) const {
    lds_trace_access(p, int(sizeof(T)), true);
    *p = v;
    return *this;
  }
};

template <typename T>
struct LdsP {
  T* p;
  LdsP(const void* q) : p(static_cast<T*>(const_cast<void*>(q))) {}
  LdsRef<T> operator*() const volatile { return LdsRef<T>{p}; }
  LdsRef<T> operator[](std::ptrdiff_t i) const volatile { return LdsRef<T>{p + i}; }
  operator T*() const volatile { return p; }
};
}  // namespace emu
