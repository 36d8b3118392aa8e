// Static device scratch of the allocation-free entry point (oomb_select_pages_noalloc).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

namespace oomb {

// Bytes of the static scratch array: the selection workspace of up to 8 MiB, i.e. the
// query-summary partials (Hkv * ceil(G*n_q/64) * D fp32), the query summaries and the
// page scores (Hkv * t0/P fp32), each rounded up to 256 bytes. The 4M-token, 8192-query
// chunk with 28/4 heads of 128 needs 2.4 MiB.
constexpr size_t kSelectScratchBytes = size_t(8) << 20;

// Device address of the scratch array on the current device. The address is looked up
// (hipGetSymbolAddress) on the first call made with each device current and kept per
// device; later calls return the kept address. Thread-safe.
hipError_t select_scratch_address(void** ptr);

}  // namespace oomb
