// Host-only stand-in for <hip/hip_runtime.h>, used solely to compile the
// library's host layer (api.cpp) with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer on a machine without a GPU.  It declares the
// few HIP runtime entities the host layer uses; stub_hip.cpp defines them
// (and the kernel launchers) without touching any device.
#pragma once

#include <stddef.h>
#include <stdint.h>

typedef enum hipError_t {
  hipSuccess = 0,
  hipErrorInvalidValue = 1,
  hipErrorNoDevice = 100,
  hipErrorInvalidDevice = 101,
  hipErrorInvalidSymbol = 13,
} hipError_t;

typedef struct ihipStream_t* hipStream_t;

typedef enum hipDeviceAttribute_t {
  hipDeviceAttributeMultiprocessorCount = 63,
} hipDeviceAttribute_t;

typedef enum hipMemcpyKind {
  hipMemcpyDeviceToHost = 2,
} hipMemcpyKind;

hipError_t hipGetDevice(int* device);
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int device);
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind kind,
                          hipStream_t stream);
hipError_t hipStreamSynchronize(hipStream_t stream);
