// Expert-bank files (plain C++, no HIP): see bank_io.cpp for the format.
#pragma once
#include <stdint.h>

#include <string>

namespace ec {

// 0 on success; -1 I/O error, -2 not a bank file of this shape (message in *err).
int bank_write(const char* path, const int32_t shape[6], int32_t pool_layers, uint64_t expert_bytes, const void* bank,
               uint64_t bytes, std::string* err);
int bank_read(const char* path, const int32_t shape[6], int32_t pool_layers, uint64_t expert_bytes, void* dst,
              uint64_t bytes, int threads, int* direct_used, double* seconds, std::string* err);

} // namespace ec
