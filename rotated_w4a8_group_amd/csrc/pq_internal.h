// Internal helpers shared by the library's translation units (host side).
#pragma once

#include <cstdint>
#include <cstddef>

#include "pq.h"

namespace pq {

// Records the message for the calling thread and returns `code`.
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Validates (P, pb1, pb2) against N. Returns PQ_OK or an error code (message set).
int check_partitions(int P, int pb1, int pb2, int N);

// Parts of the prefill GEMM's workspace (pq_gemm_workspace_bytes): the activation-side zero-point
// operand of P partitions, then the group scales transposed to [P][G][M] f32.
size_t zpe_act_bytes(int M, int G, int P);
size_t asgt_bytes(int M, int G, int P);

}  // namespace pq
