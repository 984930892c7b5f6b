// Region registry shared by the host stand-ins and the driver of the sanitized C-ABI build.
#pragma once
#include <cstddef>
#include <cstdint>
#include <cstring>
#include <string>

namespace host_abi {
extern int g_errors;
extern long g_launches;
extern float g_cos_parts[3];
void register_region(const void* base, size_t bytes, const std::string& name);
void clear_regions();
void check(const void* p, size_t bytes, const char* what);
}  // namespace host_abi
