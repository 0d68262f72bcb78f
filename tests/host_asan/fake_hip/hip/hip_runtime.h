// Host-only stand-in for the parts of the HIP runtime API that the library's
// host code (bilogp_host.cpp, bilogp_internal.h) uses, so that code can be
// built with g++ under AddressSanitizer / UndefinedBehaviorSanitizer on a
// machine without a GPU.  "Device memory" is ordinary host memory registered
// with the fake runtime (see harness.cpp); kernel launches are replaced by
// functions that touch exactly the bytes each kernel would read or write.
#pragma once

#include <stddef.h>
#include <stdint.h>

#define __device__
#define __align__(n) __attribute__((aligned(n)))
#define HIP_SYMBOL(x) ((const void*)&(x))

typedef enum hipError_t {
  hipSuccess = 0,
  hipErrorInvalidValue = 1,
  hipErrorOutOfMemory = 2,
  hipErrorNoDevice = 100,
} hipError_t;

typedef struct ihipStream_t* hipStream_t;

typedef enum hipMemoryType {
  hipMemoryTypeUnregistered = 0,
  hipMemoryTypeHost = 1,
  hipMemoryTypeDevice = 2,
  hipMemoryTypeManaged = 3,
} hipMemoryType;

typedef struct hipPointerAttribute_t {
  hipMemoryType type;
  int device;
} hipPointerAttribute_t;

typedef struct hipDeviceProp_t {
  char gcnArchName[256];
  int multiProcessorCount;
} hipDeviceProp_t;

struct float2 {
  float x, y;
};
inline float2 make_float2(float x, float y) { return float2{x, y}; }

hipError_t hipGetDevice(int* dev);
hipError_t hipGetDeviceProperties(hipDeviceProp_t* prop, int dev);
hipError_t hipPointerGetAttributes(hipPointerAttribute_t* attr, const void* ptr);
hipError_t hipGetLastError(void);
const char* hipGetErrorString(hipError_t e);
hipError_t hipMallocAsync(void** ptr, size_t bytes, hipStream_t stream);
hipError_t hipFreeAsync(void* ptr, hipStream_t stream);
hipError_t hipGetSymbolAddress(void** ptr, const void* symbol);
